"""The allocation-free entry point (packed_ctc_loss_noalloc) against packed_ctc_loss, through the C ABI.

Two allocation-free calls in a row, the second on a smaller batch, each compared with packed_ctc_loss
on the same inputs at the parity bars (losses 1e-4 relative, gradients 1e-4 absolute: float32
inputs); and a call whose workspace exceeds the library's scratch array is refused before anything
is launched.
"""

import ctypes

import numpy as np
import pytest
import torch

from ctc_forward_backward_amd import workloads as W

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ctc_forward_backward_amd import api as _api

    _api._load()
    return _api


def _call(api, b, noalloc, K=1):
    lib = api._load()
    dev = torch.device("cuda:0")
    lp, cu, ln, tg, tl = (x.to(dev) for x in (b.log_probs, b.cu_seqlens, b.lengths, b.targets, b.target_lengths))
    Umax = int(b.target_lengths.max())
    flags = 1 * (cu.dtype == torch.int64) | 2 * (ln.dtype == torch.int64) | 4 * (tg.dtype == torch.int64) \
        | 8 * (tl.dtype == torch.int64)
    losses = torch.full((b.B,), -1.0, dtype=torch.float32, device=dev)
    reduced = torch.full((), -1.0, dtype=torch.float32, device=dev)
    grad = torch.full((b.T_total, b.D), -1.0, dtype=lp.dtype, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    head = (P(lp), api.DTYPE_CODES[lp.dtype], b.T_total, b.D, P(cu), P(ln), b.B, P(tg), int(b.targets.shape[1]),
            P(tl), flags, Umax, b.blank, int(b.zero_infinity), api.REDUCTIONS[b.reduction], None, P(losses),
            P(reduced), P(grad), K)
    torch.cuda.synchronize()
    if noalloc:
        rc = lib.packed_ctc_loss_noalloc(*head, stream)
    else:
        ws_bytes = api.packed_ctc_workspace_size(b.T_total, b.D, b.B, Umax, K)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        rc = lib.packed_ctc_loss(*head, P(ws), ws_bytes, stream)
    torch.cuda.synchronize()
    assert rc == 0, lib.packed_ctc_last_error().decode()
    return losses.cpu().double().numpy(), float(reduced.cpu()), grad.cpu().double().numpy()


def test_noalloc_matches_packed_ctc_loss(api):
    _say("[gpu no-alloc] two allocation-free calls (small, then the smaller tiny) against packed_ctc_loss")
    batches = [W.make_workload("small"), W.make_workload("tiny")]
    refs = [_call(api, b, noalloc=False) for b in batches]
    gots = [_call(api, b, noalloc=True) for b in batches]  # back to back, the second smaller
    for b, (rl, rr, rg), (gl, gr, gg) in zip(batches, refs, gots):
        np.testing.assert_allclose(gl, rl, rtol=1e-4, atol=1e-5, err_msg=b.name)
        if b.reduction != "none":
            np.testing.assert_allclose(gr, rr, rtol=1e-4, atol=1e-6, err_msg=b.name)
        err = float(np.max(np.abs(gg - rg)))
        _say(f"  {b.name}: max |grad diff| = {err:.3e} (bar 1e-4)")
        assert err <= 1e-4


def test_noalloc_refuses_a_workspace_beyond_its_scratch(api):
    _say("[gpu no-alloc] a call beyond the scratch array is refused")
    b = W.make_workload("asr_bpe")  # about 810 MB of workspace
    lib = api._load()
    dev = torch.device("cuda:0")
    d = ctypes.c_void_p(0x1000)  # never dereferenced: the size check comes first
    rc = lib.packed_ctc_loss_noalloc(d, 1, b.T_total, b.D, d, d, b.B, d, int(b.targets.shape[1]), d, 8,
                                     int(b.target_lengths.max()), 0, 1, 1, None, d, d, d, 1,
                                     ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert rc == api.ERR_WORKSPACE
    assert "allocation-free" in lib.packed_ctc_last_error().decode()
    rc = lib.packed_ctc_loss_noalloc(d, 1, b.T_total, b.D, d, d, b.B, d, int(b.targets.shape[1]), d, 8, -1, 0, 1, 1,
                                     None, d, d, d, 1, ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert rc == api.ERR_ARG
