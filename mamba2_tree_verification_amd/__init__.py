"""Python binding of libssm_tree.so (argument marshalling only).

The functions ``ssm_tree_verify``, ``ssm_tree_commit``,
``ssm_tree_commit_verify``, ``ssm_tree_commit_verify_noalloc``,
``ssm_tree_plan``, ``ssm_tree_status_string`` and
``ssm_tree_abi_version`` mirror the C ABI in ``include/ssm_tree.h`` one to
one and take raw device addresses.  The ``verify`` / ``commit`` /
``commit_verify`` / ``plan`` helpers accept torch tensors on the GPU,
check their dtypes (inputs in ``dims.in_dtype``, the state in the dtype its
flag names), contiguity and element counts against the dims, raising
``ValueError`` before the library is called, pass ``data_ptr()`` and the
current HIP stream, and raise ``SsmTreeError`` on a nonzero return.  Every step of the
computation runs in the HIP kernels; there is no CPU fallback.

Debug mode: with ``SSM_TREE_DEBUG=1`` in the environment the helpers also
wait for the call to finish and raise ``SsmTreeError`` when a per-sequence
status they were given is not OK (an invalid tree or accepted path), naming
the first such sequence.  Without it, statuses are left to the caller.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssm_tree.so")

SSM_TREE_ABI_VERSION = 4
SSM_TREE_F32, SSM_TREE_BF16 = 0, 1
SSM_TREE_CONV_SILU = 1
SSM_TREE_VERIFY_FIFO = 2
SSM_TREE_CONV_XBC = 4
SSM_TREE_STATE_BF16 = 8
OK, E_NULL, E_ALIGN, E_DIMS, E_DTYPE, E_ALIAS, E_HIP, E_FLAGS, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8
E_TREE, E_PATH = -10, -11
PLAN_HEADER, PLAN_STRIDE, PLAN_UNUSED = 4, 8, -32768


class SsmTreeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, ssm_tree_status_string(code), code))
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("n_layers", "batch", "n_nodes", "nheads", "headdim", "d_state",
                                               "ngroups", "conv_width", "in_dtype", "flags")]


class Params(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("A", "D", "dt_bias", "conv_w", "conv_b")]


_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return LIB_PATH


def load():
    """Load the built library; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssm_tree.so is not built: run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        p, i = ctypes.c_void_p, ctypes.c_int
        L.ssm_tree_verify.argtypes = [p] * 13
        L.ssm_tree_verify.restype = i
        L.ssm_tree_commit.argtypes = [p] * 15
        L.ssm_tree_commit.restype = i
        L.ssm_tree_commit_verify.argtypes = [p] * 23
        L.ssm_tree_commit_verify.restype = i
        L.ssm_tree_commit_verify_noalloc.argtypes = [p] * 23
        L.ssm_tree_commit_verify_noalloc.restype = i
        L.ssm_tree_plan.argtypes = [p] * 4
        L.ssm_tree_plan.restype = i
        L.ssm_tree_status_string.argtypes = [i]
        L.ssm_tree_status_string.restype = ctypes.c_char_p
        L.ssm_tree_abi_version.argtypes = []
        L.ssm_tree_abi_version.restype = i
        if L.ssm_tree_abi_version() != SSM_TREE_ABI_VERSION:
            raise RuntimeError("libssm_tree.so ABI version mismatch")
        _lib = L
        return L


# ---------------------------------------------------------------------------
# one-to-one wrappers of the C entry points (raw addresses, ints or None)
# ---------------------------------------------------------------------------

def ssm_tree_verify(dims: Dims, params: Params, parent, x, B, C, dt_raw, z, conv_window, state, y, seq_status,
                    hip_stream) -> int:
    return load().ssm_tree_verify(ctypes.byref(dims), ctypes.byref(params), parent, x, B, C, dt_raw, z, conv_window,
                                  state, y, seq_status, hip_stream)


def ssm_tree_commit(dims: Dims, params: Params, parent, path, path_len, x, B, C, dt_raw, conv_window_in, state_in,
                    conv_window_out, state_out, seq_status, hip_stream) -> int:
    return load().ssm_tree_commit(ctypes.byref(dims), ctypes.byref(params), parent, path, path_len, x, B, C, dt_raw,
                                  conv_window_in, state_in, conv_window_out, state_out, seq_status, hip_stream)


def ssm_tree_commit_verify(dims: Dims, params: Params, parent_prev, path, path_len, x_prev, B_prev, C_prev,
                           dt_raw_prev, conv_window_in, state_in, conv_window_out, state_out, parent, x, B, C, dt_raw,
                           z, y, commit_status, verify_status, hip_stream) -> int:
    return load().ssm_tree_commit_verify(ctypes.byref(dims), ctypes.byref(params), parent_prev, path, path_len,
                                         x_prev, B_prev, C_prev, dt_raw_prev, conv_window_in, state_in,
                                         conv_window_out, state_out, parent, x, B, C, dt_raw, z, y, commit_status,
                                         verify_status, hip_stream)


def ssm_tree_commit_verify_noalloc(dims: Dims, params: Params, parent_prev, path, path_len, x_prev, B_prev, C_prev,
                                   dt_raw_prev, conv_window_in, state_in, conv_window_out, state_out, parent, x, B,
                                   C, dt_raw, z, y, commit_status, verify_status, hip_stream) -> int:
    return load().ssm_tree_commit_verify_noalloc(ctypes.byref(dims), ctypes.byref(params), parent_prev, path,
                                                 path_len, x_prev, B_prev, C_prev, dt_raw_prev, conv_window_in,
                                                 state_in, conv_window_out, state_out, parent, x, B, C, dt_raw, z, y,
                                                 commit_status, verify_status, hip_stream)


def ssm_tree_plan(dims: Dims, parent, plan_out, hip_stream) -> int:
    return load().ssm_tree_plan(ctypes.byref(dims), parent, plan_out, hip_stream)


def ssm_tree_status_string(code: int) -> str:
    try:
        return load().ssm_tree_status_string(code).decode()
    except RuntimeError:
        return "status %d" % code


def ssm_tree_abi_version() -> int:
    return load().ssm_tree_abi_version()


# ---------------------------------------------------------------------------
# torch tensor helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_dims(L, Bsz, T, H, P, N, G, W, bf16: bool, silu: bool = False, fifo: bool = False,
              xbc: bool = False, state_bf16: bool = False) -> Dims:
    return Dims(L, Bsz, T, H, P, N, G, W, SSM_TREE_BF16 if bf16 else SSM_TREE_F32,
                (SSM_TREE_CONV_SILU if silu else 0) | (SSM_TREE_VERIFY_FIFO if fifo else 0) |
                (SSM_TREE_CONV_XBC if xbc else 0) | (SSM_TREE_STATE_BF16 if state_bf16 else 0))


def make_params(A, D, dt_bias, conv_w, conv_b=None) -> Params:
    for t in (A, D, dt_bias, conv_w, conv_b):
        _check(t, "float32")
    p = Params(_ptr(A), _ptr(D), _ptr(dt_bias), _ptr(conv_w), _ptr(conv_b))
    # element counts, checked against the dims of each call
    p.numels = tuple(None if t is None else t.numel() for t in (A, D, dt_bias, conv_w, conv_b))
    return p


def _on_device(t) -> bool:
    return t.is_cuda


def _check(t, kind):
    if t is None:
        return
    import torch
    if not _on_device(t):
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    want = {"float32": (torch.float32,), "int32": (torch.int32,), "in": (torch.float32, torch.bfloat16),
            "state": (torch.float32,), "state_bf16": (torch.bfloat16,)}[kind]
    if t.dtype not in want:
        raise ValueError("unexpected dtype %s" % t.dtype)


def _state_kind(dims: Dims) -> str:
    return "state_bf16" if dims.flags & SSM_TREE_STATE_BF16 else "state"


def _sizes(dims: Dims) -> dict:
    """Element count of every tensor argument, from the layouts in
    include/ssm_tree.h."""
    L, Bsz, T, H, P, N, G, W = (dims.n_layers, dims.batch, dims.n_nodes, dims.nheads, dims.headdim, dims.d_state,
                                dims.ngroups, dims.conv_width)
    di = H * P
    ch = di + (2 * G * N if dims.flags & SSM_TREE_CONV_XBC else 0)
    U = L * Bsz
    return dict(tok=U * T * di, bc=U * T * G * N, dt=U * T * H, window=U * (W - 1) * ch, state=U * di * N,
                tree=Bsz * T, seq=Bsz, head=L * H, conv_w=L * ch * W, conv_b=L * ch)


def _check_call(dims: Dims, params: Params, items) -> None:
    """Dtype and size of every tensor of a call, before anything reaches
    the library: inputs in the dims' input dtype, the state in the dtype
    its flag names, and each element count exactly what the dims imply
    (a short tensor would otherwise be read or written past its end)."""
    import torch
    ind = torch.bfloat16 if dims.in_dtype == SSM_TREE_BF16 else torch.float32
    want = _sizes(dims)
    for name, t, kind, size in items:
        if t is None:
            continue
        _check(t, kind)
        if kind == "in" and t.dtype != ind:
            raise ValueError("%s: dtype %s, but dims.in_dtype asks for %s" % (name, t.dtype, ind))
        if size == "window" and dims.conv_width == 1:
            continue  # no window rows: never read
        if t.numel() != want[size]:
            raise ValueError("%s: %d elements, the dims imply %d" % (name, t.numel(), want[size]))
    numels = getattr(params, "numels", None)
    if numels is not None:
        for name, n, size in zip(("A", "D", "dt_bias", "conv_w", "conv_b"), numels,
                                 ("head", "head", "head", "conv_w", "conv_b")):
            if n is not None and n != want[size]:
                raise ValueError("params.%s: %d elements, the dims imply %d" % (name, n, want[size]))


def _debug() -> bool:
    return os.environ.get("SSM_TREE_DEBUG", "") not in ("", "0")


def _check_statuses(where: str, statuses) -> None:
    """Debug mode: wait for the call and raise on the first sequence whose
    status is not OK."""
    import torch
    for name, t in statuses:
        if t is None:
            continue
        if t.is_cuda:
            torch.cuda.synchronize(t.device)
        bad = (t.cpu() != OK).nonzero()
        if len(bad):
            i = int(bad[0])
            raise SsmTreeError(int(t.cpu()[i]), "%s (%s of sequence %d)" % (where, name, i))


def verify(dims: Dims, params: Params, parent, x, B, C, dt_raw, conv_window, state, y, seq_status=None,
           stream=None, z=None):
    """ssm_tree_verify; z (optional) gates y by silu(z)."""
    sk = _state_kind(dims)
    _check_call(dims, params, (("parent", parent, "int32", "tree"), ("x", x, "in", "tok"), ("B", B, "in", "bc"),
                               ("C", C, "in", "bc"), ("dt_raw", dt_raw, "in", "dt"), ("z", z, "in", "tok"),
                               ("conv_window", conv_window, "in", "window"), ("state", state, sk, "state"),
                               ("y", y, "float32", "tok"), ("seq_status", seq_status, "int32", "seq")))
    rc = ssm_tree_verify(dims, params, _ptr(parent), _ptr(x), _ptr(B), _ptr(C), _ptr(dt_raw), _ptr(z),
                         _ptr(conv_window), _ptr(state), _ptr(y), _ptr(seq_status), _stream(stream))
    if rc != OK:
        raise SsmTreeError(rc, "ssm_tree_verify")
    if _debug():
        _check_statuses("ssm_tree_verify", (("seq_status", seq_status),))


def commit(dims: Dims, params: Params, parent, path, path_len, x, B, dt_raw, conv_window_in, state_in,
           conv_window_out, state_out, seq_status=None, stream=None, C=None):
    """ssm_tree_commit; C (the raw C rows) is needed only with the xBC conv."""
    sk = _state_kind(dims)
    _check_call(dims, params, (("parent", parent, "int32", "tree"), ("path", path, "int32", "tree"),
                               ("path_len", path_len, "int32", "seq"), ("x", x, "in", "tok"), ("B", B, "in", "bc"),
                               ("C", C, "in", "bc"), ("dt_raw", dt_raw, "in", "dt"),
                               ("conv_window_in", conv_window_in, "in", "window"), ("state_in", state_in, sk, "state"),
                               ("conv_window_out", conv_window_out, "in", "window"),
                               ("state_out", state_out, sk, "state"), ("seq_status", seq_status, "int32", "seq")))
    rc = ssm_tree_commit(dims, params, _ptr(parent), _ptr(path), _ptr(path_len), _ptr(x), _ptr(B), _ptr(C),
                         _ptr(dt_raw), _ptr(conv_window_in), _ptr(state_in), _ptr(conv_window_out),
                         _ptr(state_out), _ptr(seq_status), _stream(stream))
    if rc != OK:
        raise SsmTreeError(rc, "ssm_tree_commit")
    if _debug():
        _check_statuses("ssm_tree_commit", (("seq_status", seq_status),))


def commit_verify(dims: Dims, params: Params, parent_prev, path, path_len, x_prev, B_prev, dt_raw_prev,
                  conv_window_in, state_in, conv_window_out, state_out, parent, x, B, C, dt_raw, y,
                  commit_status=None, verify_status=None, stream=None, C_prev=None, z=None, noalloc=False):
    """ssm_tree_commit_verify; C_prev is needed only with the xBC conv, z
    (optional) gates the next tree's y by silu(z); noalloc calls
    ssm_tree_commit_verify_noalloc instead (no allocation; its fixed scratch
    is shared by every such call on the device)."""
    sk = _state_kind(dims)
    _check_call(dims, params, (("parent_prev", parent_prev, "int32", "tree"), ("path", path, "int32", "tree"),
                               ("path_len", path_len, "int32", "seq"), ("x_prev", x_prev, "in", "tok"),
                               ("B_prev", B_prev, "in", "bc"), ("C_prev", C_prev, "in", "bc"),
                               ("dt_raw_prev", dt_raw_prev, "in", "dt"),
                               ("conv_window_in", conv_window_in, "in", "window"), ("state_in", state_in, sk, "state"),
                               ("conv_window_out", conv_window_out, "in", "window"),
                               ("state_out", state_out, sk, "state"), ("parent", parent, "int32", "tree"),
                               ("x", x, "in", "tok"), ("B", B, "in", "bc"), ("C", C, "in", "bc"),
                               ("dt_raw", dt_raw, "in", "dt"), ("z", z, "in", "tok"), ("y", y, "float32", "tok"),
                               ("commit_status", commit_status, "int32", "seq"),
                               ("verify_status", verify_status, "int32", "seq")))
    fn = ssm_tree_commit_verify_noalloc if noalloc else ssm_tree_commit_verify
    rc = fn(dims, params, _ptr(parent_prev), _ptr(path), _ptr(path_len), _ptr(x_prev),
                                _ptr(B_prev), _ptr(C_prev), _ptr(dt_raw_prev), _ptr(conv_window_in),
                                _ptr(state_in), _ptr(conv_window_out), _ptr(state_out), _ptr(parent), _ptr(x),
                                _ptr(B), _ptr(C), _ptr(dt_raw), _ptr(z), _ptr(y), _ptr(commit_status),
                                _ptr(verify_status), _stream(stream))
    if rc != OK:
        raise SsmTreeError(rc, "ssm_tree_commit_verify_noalloc" if noalloc else "ssm_tree_commit_verify")
    if _debug():
        _check_statuses("ssm_tree_commit_verify", (("commit_status", commit_status), ("verify_status", verify_status)))


def plan(dims: Dims, parent, plan_out, stream=None):
    _check(parent, "int32")
    _check(plan_out, "int32")
    if parent is not None and parent.numel() != dims.batch * dims.n_nodes:
        raise ValueError("parent: %d elements, the dims imply %d" % (parent.numel(), dims.batch * dims.n_nodes))
    want = dims.batch * (PLAN_HEADER + dims.n_nodes * PLAN_STRIDE)
    if plan_out is not None and plan_out.numel() != want:
        raise ValueError("plan_out: %d elements, the dims imply %d" % (plan_out.numel(), want))
    rc = ssm_tree_plan(dims, _ptr(parent), _ptr(plan_out), _stream(stream))
    if rc != OK:
        raise SsmTreeError(rc, "ssm_tree_plan")
