"""The torch helpers refuse, before the library is called, tensors whose
dtype or element count does not match the dims (CPU only: the device check
is bypassed so that host tensors stand in for device ones, and every call
here fails on a check before any pointer is used).  Debug mode
(SSM_TREE_DEBUG=1) is checked with the entry points replaced by stubs that
return OK."""
import pytest

torch = pytest.importorskip("torch")
import mamba2_tree_verification_amd as m  # noqa: E402

L, BSZ, T, H, P, N, G, W = 2, 3, 5, 4, 16, 16, 1, 4
DI = H * P


@pytest.fixture(autouse=True)
def host_tensors_pass_device_check(monkeypatch):
    monkeypatch.setattr(m, "_on_device", lambda t: True)

    def no_library(*a, **k):
        raise AssertionError("a refused call reached the library")

    for f in ("ssm_tree_verify", "ssm_tree_commit", "ssm_tree_commit_verify", "ssm_tree_plan"):
        monkeypatch.setattr(m, f, no_library)


def dims(bf16=True, xbc=False, state_bf16=False):
    return m.make_dims(L, BSZ, T, H, P, N, G, W, bf16, xbc=xbc, state_bf16=state_bf16)


def inputs(bf16=True, xbc=False, state_bf16=False):
    e = torch.bfloat16 if bf16 else torch.float32
    ch = DI + (2 * G * N if xbc else 0)
    return dict(
        parent=torch.zeros(BSZ, T, dtype=torch.int32), path=torch.zeros(BSZ, T, dtype=torch.int32),
        path_len=torch.zeros(BSZ, dtype=torch.int32), x=torch.zeros(L, BSZ, T, DI, dtype=e),
        B=torch.zeros(L, BSZ, T, G, N, dtype=e), C=torch.zeros(L, BSZ, T, G, N, dtype=e),
        dt_raw=torch.zeros(L, BSZ, T, H, dtype=e), z=torch.zeros(L, BSZ, T, DI, dtype=e),
        window=torch.zeros(L, BSZ, W - 1, ch, dtype=e),
        state=torch.zeros(L, BSZ, H, P, N, dtype=torch.bfloat16 if state_bf16 else torch.float32),
        y=torch.zeros(L, BSZ, T, DI), status=torch.zeros(BSZ, dtype=torch.int32),
        A=torch.zeros(L, H), D=torch.zeros(L, H), dt_bias=torch.zeros(L, H), conv_w=torch.zeros(L, ch, W))


def params(t, **over):
    a = dict(A=t["A"], D=t["D"], dt_bias=t["dt_bias"], conv_w=t["conv_w"])
    a.update(over)
    return m.make_params(a["A"], a["D"], a["dt_bias"], a["conv_w"], a.get("conv_b"))


def call_verify(d, t, prm=None, **over):
    a = dict(t)
    a.update(over)
    m.verify(d, prm or params(t), a["parent"], a["x"], a["B"], a["C"], a["dt_raw"], a["window"], a["state"], a["y"],
             a["status"], z=a.get("zz"))


def call_commit(d, t, prm=None, **over):
    a = dict(t)
    a.update(over)
    m.commit(d, prm or params(t), a["parent"], a["path"], a["path_len"], a["x"], a["B"], a["dt_raw"], a["window"],
             a["state"], a.get("win_out", a["window"]), a.get("state_out", a["state"]), a["status"])


def call_round(d, t, prm=None, **over):
    a = dict(t)
    a.update(over)
    m.commit_verify(d, prm or params(t), a["parent"], a["path"], a["path_len"], a["x"], a["B"], a["dt_raw"],
                    a["window"], a["state"], a["window"], a["state"], a["parent"], a.get("x_next", a["x"]), a["B"],
                    a["C"], a["dt_raw"], a["y"], a["status"], a.get("vstatus", a["status"]))


@pytest.mark.parametrize("name,bad", [
    ("x", lambda t: t["x"][..., :-1].contiguous()), ("B", lambda t: t["B"][:1].contiguous()),
    ("C", lambda t: t["C"][:, :2].contiguous()), ("dt_raw", lambda t: t["dt_raw"][..., :1].contiguous()),
    ("window", lambda t: t["window"][:, :, :1].contiguous()), ("state", lambda t: t["state"][:1].contiguous()),
    ("y", lambda t: t["y"][:, :, :2].contiguous()), ("parent", lambda t: t["parent"][:, :2].contiguous()),
    ("status", lambda t: t["status"][:1].contiguous())])
def test_verify_refuses_short_tensors(name, bad):
    t = inputs()
    with pytest.raises(ValueError, match="elements"):
        call_verify(dims(), t, **{name: bad(t)})


@pytest.mark.parametrize("name,bad", [
    ("path", lambda t: t["path"][:, :1].contiguous()), ("path_len", lambda t: t["path_len"][:2].contiguous()),
    ("x", lambda t: t["x"][:1].contiguous()), ("state_out", lambda t: t["state"][:, :2].contiguous()),
    ("win_out", lambda t: t["window"][:, :, :2].contiguous())])
def test_commit_refuses_short_tensors(name, bad):
    t = inputs()
    with pytest.raises(ValueError, match="elements"):
        call_commit(dims(), t, **{name: bad(t)})


def test_round_refuses_short_tensors():
    t = inputs()
    with pytest.raises(ValueError, match="elements"):
        call_round(dims(), t, x_next=t["x"][:, :, :2].contiguous())
    with pytest.raises(ValueError, match="elements"):
        call_round(dims(), t, vstatus=torch.zeros(BSZ + 1, dtype=torch.int32))


def test_inputs_must_be_in_the_dims_dtype():
    t = inputs(bf16=False)
    with pytest.raises(ValueError, match="in_dtype"):
        call_verify(dims(bf16=True), t)
    t = inputs(bf16=True)
    with pytest.raises(ValueError, match="in_dtype"):
        call_commit(dims(bf16=False), t)
    t = inputs(bf16=True)
    with pytest.raises(ValueError, match="in_dtype"):
        call_round(dims(), t, x_next=t["x"].float())


def test_state_dtype_follows_its_flag():
    t = inputs(state_bf16=True)
    with pytest.raises(ValueError, match="dtype"):
        call_verify(dims(state_bf16=False), t)
    t = inputs(state_bf16=False)
    with pytest.raises(ValueError, match="dtype"):
        call_commit(dims(state_bf16=True), t)


def test_params_sizes_follow_the_dims():
    t = inputs()
    with pytest.raises(ValueError, match="params.A"):
        call_verify(dims(), t, prm=params(t, A=torch.zeros(L, H - 1)))
    with pytest.raises(ValueError, match="params.conv_w"):
        call_commit(dims(), t, prm=params(t, conv_w=torch.zeros(L, DI, W - 1)))
    # the xBC conv widens the window and the conv weights to d_in + 2GN channels
    tx = inputs(xbc=True)
    with pytest.raises(ValueError, match="params.conv_b"):
        call_verify(dims(xbc=True), tx, prm=params(tx, conv_b=torch.zeros(L, DI)))
    with pytest.raises(ValueError, match="conv_window"):
        call_verify(dims(xbc=True), dict(tx, window=t["window"]))


def test_plan_sizes():
    d = dims()
    with pytest.raises(ValueError, match="plan_out"):
        m.plan(d, torch.zeros(BSZ, T, dtype=torch.int32), torch.zeros(BSZ * (m.PLAN_HEADER + T * m.PLAN_STRIDE) - 1,
                                                                     dtype=torch.int32))
    with pytest.raises(ValueError, match="parent"):
        m.plan(d, torch.zeros(BSZ, T - 1, dtype=torch.int32),
               torch.zeros(BSZ * (m.PLAN_HEADER + T * m.PLAN_STRIDE), dtype=torch.int32))


def _returns_ok(*a, **k):
    return m.OK


def test_debug_mode_raises_on_a_failed_sequence(monkeypatch):
    """SSM_TREE_DEBUG=1: a call that returns OK but leaves a sequence's
    status at E_TREE raises and names that sequence; without it the status is
    left to the caller."""
    monkeypatch.setattr(m, "ssm_tree_verify", _returns_ok)
    monkeypatch.setattr(m, "ssm_tree_commit_verify", _returns_ok)
    monkeypatch.setattr(m, "_stream", lambda s: 0)
    t = inputs()
    t["status"][1] = m.E_TREE
    monkeypatch.delenv("SSM_TREE_DEBUG", raising=False)
    call_verify(dims(), t)
    monkeypatch.setenv("SSM_TREE_DEBUG", "1")
    with pytest.raises(m.SsmTreeError, match="sequence 1") as e:
        call_verify(dims(), t)
    assert e.value.code == m.E_TREE
    t["status"][1] = m.OK
    call_verify(dims(), t)
    # the round: either status names the sequence
    st2 = torch.zeros(BSZ, dtype=torch.int32)
    st2[2] = m.E_PATH
    with pytest.raises(m.SsmTreeError, match="commit_status of sequence 2"):
        m.commit_verify(dims(), params(t), t["parent"], t["path"], t["path_len"], t["x"], t["B"], t["dt_raw"],
                        t["window"], t["state"], t["window"], t["state"], t["parent"], t["x"], t["B"], t["C"],
                        t["dt_raw"], t["y"], st2, t["status"])
