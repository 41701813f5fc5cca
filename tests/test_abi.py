"""The C ABI without a GPU: the library loads, exports every declared symbol, sizes workspaces, and
rejects bad arguments with the documented error codes before anything is launched."""

import ctypes
import os
import re

import pytest
import torch

from ctc_forward_backward_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "packed_ctc.h")


def _declared_functions():
    import glob

    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\w[\w\s\*]*?\b((?:packed_ctc|hmm)_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("packed_ctc_loss", "packed_ctc_reduce", "packed_ctc_workspace_size", "packed_ctc_last_error",
              "packed_ctc_max_target_length", "packed_ctc_limits", "packed_ctc_version",
              "packed_ctc_set_phase_timing", "packed_ctc_phase_times", "packed_ctc_workspace_status",
              "packed_ctc_forward", "packed_ctc_backward", "hmm_forward_loglik", "packed_ctc_set_pipeline",
              "packed_ctc_pipeline"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(api.library_path())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_error_code_values_match_header():
    src = open(HEADER).read()
    codes = dict(re.findall(r"#define (PCTC_(?:OK|ERR_\w+))\s+(\d+)", src))
    assert int(codes["PCTC_OK"]) == api.OK
    assert int(codes["PCTC_ERR_SHAPE"]) == api.ERR_SHAPE
    assert int(codes["PCTC_ERR_DTYPE"]) == api.ERR_DTYPE
    assert int(codes["PCTC_ERR_BLANK"]) == api.ERR_BLANK
    assert int(codes["PCTC_ERR_NEG_TARGET_LENGTH"]) == api.ERR_NEG
    assert int(codes["PCTC_ERR_TARGET_LENGTH_WIDTH"]) == api.ERR_WIDTH
    assert int(codes["PCTC_ERR_WORKSPACE"]) == api.ERR_WORKSPACE
    assert int(codes["PCTC_ERR_HIP"]) == api.ERR_HIP
    assert int(codes["PCTC_ERR_ARG"]) == api.ERR_ARG
    assert int(codes["PCTC_ERR_LIMIT"]) == api.ERR_LIMIT


def test_workspace_size():
    f = api.packed_ctc_workspace_size
    assert f(0, 5, 0, 0) >= 0
    a = f(1000, 1025, 8, 100)
    assert a > 0 and a % 256 == 0
    assert f(2000, 1025, 8, 100) > a
    assert f(1000, 1025, 8, 200) > a
    # the alpha and beta tables dominate: at least 2 * T_total * (2U + 2) floats
    assert a >= 2 * 1000 * 202 * 4
    lib = api._load()
    assert lib.packed_ctc_workspace_size(-1, 5, 1, 1, 1) == 0
    assert lib.packed_ctc_workspace_size(5, 5, 1, -1, 1) == 0
    assert lib.packed_ctc_workspace_size(5, 5, 1, 1, 3) == 0
    assert lib.packed_ctc_workspace_size(5, 5, 1, 1, 64) == 0
    # alpha checkpointing: the alpha part shrinks about K-fold; beta and the rest stay
    full = f(32839, 8193, 16, 490)
    k32 = f(32839, 8193, 16, 490, 32)
    alpha = 8 * 32839 * 512  # Gmax = 8 blocks of 128 floats per row
    assert full - k32 >= 0.9 * alpha
    assert f(32839, 8193, 16, 490, 8) > k32


def test_limits_and_version():
    u, d = api.limits()
    assert u >= 3000 and d >= 8193
    assert b"gfx950" in api._load().packed_ctc_version()


def _call(**kw):
    """packed_ctc_loss with dummy (never dereferenced) pointers; every case fails in the host checks."""
    lib = api._load()
    dummy = ctypes.c_void_p(0x1000)
    a = dict(log_probs=dummy, dtype=0, T_total=10, D=5, cu=dummy, lengths=dummy, B=2, targets=dummy, W=3,
             tl=dummy, flags=0, maxU=3, blank=0, zi=0, red=0, gs=None, losses=dummy, reduced=None, grad=None,
             K=1, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.packed_ctc_loss(a["log_probs"], a["dtype"], a["T_total"], a["D"], a["cu"], a["lengths"], a["B"],
                               a["targets"], a["W"], a["tl"], a["flags"], a["maxU"], a["blank"], a["zi"], a["red"],
                               a["gs"], a["losses"], a["reduced"], a["grad"], a["K"], a["ws"], a["ws_bytes"],
                               a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(T_total=-1), api.ERR_SHAPE, "shape"),
    (dict(D=-3), api.ERR_SHAPE, "shape"),
    (dict(dtype=4), api.ERR_DTYPE, "float32"),
    (dict(dtype=7), api.ERR_DTYPE, "float32"),
    (dict(B=-1), api.ERR_SHAPE, "batch"),
    (dict(W=-1), api.ERR_SHAPE, "width"),
    (dict(blank=5), api.ERR_BLANK, "blank"),
    (dict(blank=-1), api.ERR_BLANK, "blank"),
    (dict(red=3), api.ERR_ARG, "reduction"),
    (dict(flags=16), api.ERR_ARG, "flags"),
    (dict(log_probs=None), api.ERR_ARG, "log_probs"),
    (dict(cu=None), api.ERR_ARG, "required"),
    (dict(losses=None), api.ERR_ARG, "required"),
    (dict(targets=None), api.ERR_ARG, "targets"),
    (dict(log_probs=ctypes.c_void_p(0x1008)), api.ERR_ARG, "aligned"),
    (dict(grad=ctypes.c_void_p(0x1004)), api.ERR_ARG, "aligned"),
    (dict(maxU=9000, W=9000), api.ERR_LIMIT, "limit"),
    (dict(D=40000, grad=ctypes.c_void_p(0x1000)), api.ERR_LIMIT, "limit"),
    (dict(ws=None, ws_bytes=0), api.ERR_WORKSPACE, "workspace"),
    (dict(ws=ctypes.c_void_p(0x1000), ws_bytes=16), api.ERR_WORKSPACE, "workspace"),
    (dict(ws=ctypes.c_void_p(0x1001), ws_bytes=1 << 40), api.ERR_WORKSPACE, "aligned"),
    (dict(K=3), api.ERR_ARG, "checkpoint_interval"),
    (dict(K=64), api.ERR_ARG, "checkpoint_interval"),
    (dict(K=0), api.ERR_ARG, "checkpoint_interval"),
    (dict(K=8, dtype=3), api.ERR_ARG, "checkpointing"),
    (dict(K=8, maxU=1024, W=1024), api.ERR_LIMIT, "checkpointing"),
])
def test_host_checks(kw, code, needle):
    rc = _call(**kw)
    assert rc == code
    assert needle in api._load().packed_ctc_last_error().decode()


def test_reduce_host_checks():
    lib = api._load()
    d = ctypes.c_void_p(0x1000)
    assert lib.packed_ctc_reduce(d, d, 0, 4, 0, d, None) == api.ERR_ARG
    assert lib.packed_ctc_reduce(d, d, 0, -1, 1, d, None) == api.ERR_SHAPE
    assert lib.packed_ctc_reduce(d, d, 0, 4, 1, None, None) == api.ERR_ARG


def test_binding_checks_without_gpu():
    lp = torch.zeros(10, 5)
    args = (torch.tensor([0, 6, 10], dtype=torch.int32), torch.tensor([6, 4]), torch.zeros(2, 2, dtype=torch.long),
            torch.tensor([1, 2]))
    with pytest.raises(ValueError, match="shape"):
        api.packed_ctc_loss(torch.zeros(2, 5, 5), *args, blank=0)
    with pytest.raises(RuntimeError, match="GPU"):
        api.packed_ctc_loss(lp, *args, blank=0)


def _split(which, **kw):
    """packed_ctc_forward / packed_ctc_backward with dummy pointers; every case fails in the host checks."""
    lib = api._load()
    dummy = ctypes.c_void_p(0x1000)
    a = dict(log_probs=dummy, dtype=0, T_total=10, D=5, cu=dummy, lengths=dummy, B=2, targets=dummy, W=3,
             tl=dummy, flags=0, maxU=3, blank=0, zi=0, red=0, gs=None, losses=dummy, reduced=None, grad=dummy,
             K=1, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    head = (a["log_probs"], a["dtype"], a["T_total"], a["D"], a["cu"], a["lengths"], a["B"], a["targets"], a["W"],
            a["tl"], a["flags"], a["maxU"], a["blank"], a["zi"], a["red"])
    if which == "forward":
        return lib.packed_ctc_forward(*head, a["losses"], a["reduced"], a["K"], a["ws"], a["ws_bytes"], a["stream"])
    return lib.packed_ctc_backward(*head, a["gs"], a["grad"], a["K"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("which,kw,code,needle", [
    ("forward", dict(dtype=4), api.ERR_DTYPE, "float32"),
    ("forward", dict(blank=7), api.ERR_BLANK, "blank"),
    ("forward", dict(losses=None), api.ERR_ARG, "required"),
    ("forward", dict(ws=None, ws_bytes=0), api.ERR_WORKSPACE, "workspace"),
    ("backward", dict(maxU=-1), api.ERR_ARG, "max_target_length"),
    ("backward", dict(grad=None), api.ERR_ARG, "grad_out"),
    ("backward", dict(grad=ctypes.c_void_p(0x1004)), api.ERR_ARG, "aligned"),
    ("backward", dict(red=5), api.ERR_ARG, "reduction"),
    ("backward", dict(ws=ctypes.c_void_p(0x1000), ws_bytes=16), api.ERR_WORKSPACE, "workspace"),
])
def test_split_entry_points_host_checks(which, kw, code, needle):
    rc = _split(which, **kw)
    assert rc == code
    assert needle in api._load().packed_ctc_last_error().decode()


def test_autograd_binding_checks_without_gpu():
    lp = torch.zeros(10, 5, requires_grad=True)
    args = (torch.tensor([0, 6, 10], dtype=torch.int32), torch.tensor([6, 4]), torch.zeros(2, 2, dtype=torch.long),
            torch.tensor([1, 2]))
    with pytest.raises(RuntimeError, match="GPU"):
        api.ctc_loss(lp, *args, blank=0)
    with pytest.raises(ValueError, match="shape"):
        api.ctc_loss(torch.zeros(2, 5, 5, requires_grad=True), *args, blank=0)



@pytest.mark.parametrize("kw,code,needle", [
    (dict(B=-1), api.ERR_SHAPE, "batch"),
    (dict(S=0), api.ERR_LIMIT, "states"),
    (dict(S=65), api.ERR_LIMIT, "states"),
    (dict(O=0), api.ERR_LIMIT, "S * O"),
    (dict(S=64, O=300), api.ERR_LIMIT, "S * O"),
    (dict(T=0), api.ERR_SHAPE, "frame"),
    (dict(i64=2), api.ERR_ARG, "observations_i64"),
    (dict(out=None), api.ERR_ARG, "NULL"),
])
def test_hmm_host_checks(kw, code, needle):
    lib = api._load()
    d = ctypes.c_void_p(0x1000)
    a = dict(B=4, T=8, S=16, O=64, i64=0, out=d)
    a.update(kw)
    rc = lib.hmm_forward_loglik(d, d, d, d, a["i64"], a["B"], a["T"], a["S"], a["O"], a["out"], None)
    assert rc == code
    assert needle in lib.packed_ctc_last_error().decode()


def test_pipeline_switch():
    """The pipeline choice is host state only: set, read back, unknown values rejected."""
    src = open(HEADER).read()
    codes = dict(re.findall(r"#define (PCTC_PIPELINE_\w+)\s+(\d+)", src))
    assert {k: int(v) for k, v in codes.items()} == {"PCTC_PIPELINE_GROUPED": 0, "PCTC_PIPELINE_STREAMED": 1}
    lib = api._load()
    before = api.pipeline()
    assert before == "streamed"  # the default
    try:
        api.set_pipeline("grouped")
        assert api.pipeline() == "grouped" and lib.packed_ctc_pipeline() == 0
        api.set_pipeline("streamed")
        assert lib.packed_ctc_pipeline() == 1
        assert lib.packed_ctc_set_pipeline(7) == api.ERR_ARG
        assert "unknown pipeline" in lib.packed_ctc_last_error().decode()
        assert api.pipeline() == "streamed"
        with pytest.raises(ValueError):
            api.set_pipeline("fast")
    finally:
        api.set_pipeline(before)
