"""The split entry points (packed_ctc_forward / packed_ctc_backward), the autograd binding and graph
capture, on the GPU, through the C ABI.

- The split call gives the fused call's losses and gradient (the same kernels; float32 workloads,
  within 1e-6, since class sums are accumulated with LDS atomics in no fixed order).
- The backward with upstream weights in [-1, 1] matches the float64 oracle with those weights as
  grad_scale, at the parity tolerances (losses 1e-4 / 2e-3 relative, gradients 1e-4 / 2e-3
  absolute for float32 / 16-bit inputs); a second backward on the same forward state matches as
  well.
- Autograd (`ctc_loss` + `.backward`) for none / sum / mean matches the oracle.
- The forward that writes the gradient too (packed_ctc_forward_grad): with unit upstream weights the
  update leaves it as the fused call wrote it (the same bytes, also through autograd's
  `loss.backward()`); other weights rewrite it to the oracle's, and a later update with unit
  weights rewrites it again; on both pipelines, at checkpoint interval 8 and for float64.
- A captured graph of the fused call and one of the autograd forward + backward, with the target
  bound set to the targets width (no host read), replayed several times on fresh inputs with eager
  work between replays: every replay matches an eager call on the same inputs.
- The page's graph-replay scenario (PR page, test file, `test_cuda_graph_replay`), with seeded
  values of our own: a capture sized by the targets width, then replays after new targets, target
  lengths and frame lengths are copied into the captured buffers (a target as long as the width,
  empty targets, a zero-length utterance, junk past every length); each replay is compared with
  the float64 oracle on that replay's metadata, on both pipelines of the fused call and through
  autograd.
"""

import numpy as np
import pytest
import torch

from ctc_forward_backward_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-4, 1e-4), torch.bfloat16: (2e-3, 2e-3), torch.float16: (2e-3, 2e-3),
       torch.float64: (1e-10, 1e-10)}


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ctc_forward_backward_amd import api as _api

    _api._load()
    return _api


def _dev_args(b):
    dev = torch.device("cuda:0")
    return (b.cu_seqlens.to(dev), b.lengths.to(dev), b.targets.to(dev), b.target_lengths.to(dev))


def _check_oracle(losses, grad, ref, dtype, label):
    """The parity bar: losses within 1e-4 / 2e-3 relative, gradients within 1e-4 / 2e-3 absolute
    (float32 / 16-bit inputs).  The upstream weights of these tests lie in [-1, 1], so every
    gradient entry stays within the unit-weight range the bar is set for."""
    lrt, gat = TOL[dtype]
    loss = losses.detach().cpu().double().numpy()
    rloss = ref["loss"]
    assert np.array_equal(np.isinf(loss), np.isinf(rloss)), label
    fin = ~np.isinf(rloss)
    np.testing.assert_allclose(loss[fin], rloss[fin], rtol=lrt, atol=0 if dtype == torch.float64 else 1e-5,
                               err_msg=label)
    if grad is not None:
        g = grad.detach().cpu().double().numpy()
        rg = ref["grad"]
        nan_ref = np.isnan(rg)
        assert np.array_equal(np.isnan(g), nan_ref), label
        err = np.abs(g - rg)[~nan_ref]
        worst = float(err.max()) if err.size else 0.0
        _say(f"  {label}: max |grad err| = {worst:.3e} (tol {gat})")
        assert worst <= gat, f"{label}: gradient error {worst} > {gat}"


@pytest.mark.parametrize("name", ["small", "char_level"])
def test_split_matches_fused(api, name):
    _say(f"[gpu autograd] split vs fused, workload {name}")
    b = W.make_workload(name)
    lp = b.log_probs.to("cuda:0")
    args = _dev_args(b)
    kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction)
    l1, r1, g1 = api.packed_ctc_loss(lp, *args, **kw)
    l2, r2, state = api.packed_ctc_forward(lp, *args, **kw)
    g2 = api.packed_ctc_backward(state, zero_infinity=b.zero_infinity)
    torch.cuda.synchronize()
    assert api.last_call_status() == 0
    assert torch.allclose(l1, l2, rtol=1e-6, atol=0), name
    assert torch.allclose(r1, r2, rtol=1e-6, atol=0), name
    assert float((g1.double() - g2.double()).abs().max()) <= 1e-6, name


@pytest.mark.parametrize("name", ["tiny", "asr_bpe", "large_vocab"])
def test_backward_weights_vs_oracle(api, oracle_mod, name):
    _say(f"[gpu autograd] backward with upstream weights, workload {name}")
    b = W.make_workload(name)
    lp = b.log_probs.to("cuda:0")
    losses, _, state = api.packed_ctc_forward(lp, *_dev_args(b), blank=b.blank, zero_infinity=b.zero_infinity,
                                              reduction="none")
    rng = np.random.default_rng(21)
    for k in range(2):  # the same forward state serves two backward calls
        gs = rng.uniform(-1.0, 1.0, size=b.B).astype(np.float32)
        gs[0] = 0.0
        grad = api.packed_ctc_backward(state, torch.from_numpy(gs), zero_infinity=b.zero_infinity, reduction="none")
        torch.cuda.synchronize()
        ref = oracle_mod.ctc_batch(b, reduction="none", grad_scale=gs.astype(np.float64))
        _check_oracle(losses, grad, ref, b.log_probs.dtype, f"{name}/backward {k}")
    assert api.last_call_status() == 0


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_autograd_vs_oracle(api, oracle_mod, reduction):
    _say(f"[gpu autograd] ctc_loss.backward, reduction {reduction}")
    b = W.make_workload("small")
    lp = b.log_probs.to("cuda:0").requires_grad_(True)
    out = api.ctc_loss(lp, *_dev_args(b), blank=b.blank, zero_infinity=b.zero_infinity, reduction=reduction)
    if reduction == "none":
        g = torch.linspace(-1.0, 1.0, b.B, dtype=torch.float32, device="cuda:0")
        out.backward(g)
        gs = g.cpu().double().numpy()
    else:
        assert out.ndim == 0
        out.backward(torch.tensor(0.75, device="cuda:0"))
        gs = np.full(b.B, 0.75)
    torch.cuda.synchronize()
    ref = oracle_mod.ctc_batch(b, reduction=reduction, grad_scale=gs)
    losses = out if reduction == "none" else torch.from_numpy(ref["loss"])  # scalar checked below
    _check_oracle(losses, lp.grad, ref, b.log_probs.dtype, f"autograd/{reduction}")
    if reduction != "none":
        np.testing.assert_allclose(float(out.detach().cpu()), ref["reduced"], rtol=1e-4)
    assert lp.grad.dtype == lp.dtype


@pytest.mark.parametrize("case", ["small/streamed", "asr_bpe/grouped", "large_vocab/streamed", "small/K8",
                                  "float64"])
def test_forward_grad_and_update(api, oracle_mod, case):
    _say(f"[gpu autograd] forward with the gradient, then updates: {case}")
    name, how = case.split("/") if "/" in case else ("small", case)
    b = W.make_workload(name)
    if how == "float64":
        b = W.make_batch([300, 41, 0, 170], [[1, 2, 2, 3], [4], [5], [6, 1, 6]], 9, seed=5, sigma=1.5, dtype="f64",
                         reduction="mean")
    lp = b.log_probs.to("cuda:0")
    args = _dev_args(b)
    K = 8 if how == "K8" else 1
    kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction,
              max_target_length=int(b.target_lengths.max()), checkpoint_interval=K)
    old = api.pipeline()
    api.set_pipeline("grouped" if how == "grouped" else "streamed")
    try:
        l0, r0, _ = api.packed_ctc_loss(lp, *args, **kw)
        losses, reduced, grad, state = api.packed_ctc_forward_grad(lp, *args, **kw)
        torch.cuda.synchronize()
        assert api.last_call_status() == 0
        assert torch.equal(losses, l0) and (reduced is None or torch.equal(reduced, r0)), case
        unit_ref = oracle_mod.ctc_batch(b, reduction=b.reduction)
        _check_oracle(losses, grad, unit_ref, lp.dtype, f"{case}/forward")
        ones = torch.ones(b.B, dtype=losses.dtype)
        first = grad.clone()
        api.packed_ctc_backward_update(state, ones, grad, zero_infinity=b.zero_infinity)
        torch.cuda.synchronize()
        assert torch.equal(grad, first), f"{case}: a unit update changed the rows"
        rng = np.random.default_rng(5)
        gs = rng.uniform(-1.0, 1.0, size=b.B)
        gs[0] = 0.0
        api.packed_ctc_backward_update(state, torch.from_numpy(gs).to(losses.dtype), grad,
                                       zero_infinity=b.zero_infinity)
        torch.cuda.synchronize()
        ref = oracle_mod.ctc_batch(b, reduction=b.reduction, grad_scale=gs)
        _check_oracle(losses, grad, ref, lp.dtype, f"{case}/update")
        # after other weights, unit weights rewrite the rows (the forward's are gone)
        api.packed_ctc_backward_update(state, ones, grad, zero_infinity=b.zero_infinity)
        torch.cuda.synchronize()
        _check_oracle(losses, grad, unit_ref, lp.dtype, f"{case}/unit again")
        assert api.last_call_status() == 0
    finally:
        api.set_pipeline(old)


def test_autograd_unit_upstream_keeps_the_forward_rows(api, oracle_mod):
    _say("[gpu autograd] loss.backward() with the forward's rows")
    b = W.make_workload("large_vocab")
    lp0 = b.log_probs.to("cuda:0")
    kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction)
    _, _, fused = api.packed_ctc_loss(lp0, *_dev_args(b), **kw)
    lp = lp0.clone().requires_grad_(True)
    out = api.ctc_loss(lp, *_dev_args(b), **kw)
    out.backward()
    torch.cuda.synchronize()
    assert api.last_call_status() == 0
    tol = TOL[lp.dtype][1]
    assert float((lp.grad.double() - fused.double()).abs().max()) <= tol
    ref = oracle_mod.ctc_batch(b)
    _check_oracle(torch.from_numpy(ref["loss"]), lp.grad, ref, lp.dtype, "autograd/unit")
    # a tensor that needs no gradient: the loss only
    out2 = api.ctc_loss(lp0, *_dev_args(b), **kw)
    torch.cuda.synchronize()
    assert torch.allclose(out2, out.detach(), rtol=1e-6, atol=0)


def _fresh_lp(b, k):
    rng = np.random.default_rng(100 + k)
    logits = rng.normal(0.0, 2.0, size=tuple(b.log_probs.shape))
    lp = logits - np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1, keepdims=True)) - logits.max(1, keepdims=True)
    return torch.from_numpy(lp).to(b.log_probs.dtype)


def test_graph_capture_fused_call(api):
    _say("[gpu autograd] graph capture of the fused call")
    b = W.make_workload("small")
    dev = torch.device("cuda:0")
    args = _dev_args(b)
    Wd = int(b.targets.shape[1])
    kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction, max_target_length=Wd)
    lp_static = b.log_probs.to(dev).clone()
    api.packed_ctc_loss(lp_static, *args, **kw)  # eager first: the library's group streams exist
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        losses, reduced, grad = api.packed_ctc_loss(lp_static, *args, **kw)
    for k in range(3):
        fresh = _fresh_lp(b, k).to(dev)
        lp_static.copy_(fresh)
        graph.replay()
        torch.cuda.synchronize()
        el, er, eg = api.packed_ctc_loss(fresh, *args, **kw)  # eager work between replays
        torch.cuda.synchronize()
        assert api.last_call_status() == 0
        assert torch.allclose(losses, el, rtol=1e-6, atol=0), k
        assert torch.allclose(reduced, er, rtol=1e-6, atol=0), k
        assert float((grad.double() - eg.double()).abs().max()) <= 1e-6, k
        _say(f"  replay {k}: matches the eager call")


def test_graph_capture_autograd(api):
    _say("[gpu autograd] graph capture of ctc_loss forward + backward")
    b = W.make_workload("small")
    dev = torch.device("cuda:0")
    args = _dev_args(b)
    Wd = int(b.targets.shape[1])
    kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction="mean", max_target_length=Wd)
    lp_static = b.log_probs.to(dev).clone().requires_grad_(True)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm-up outside the capture, as torch asks
        for _ in range(2):
            lp_static.grad = None
            api.ctc_loss(lp_static, *args, **kw).backward()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    lp_static.grad = None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = api.ctc_loss(lp_static, *args, **kw)
        out.backward()
    for k in range(3):
        fresh = _fresh_lp(b, 10 + k).to(dev)
        with torch.no_grad():
            lp_static.copy_(fresh)
        graph.replay()
        torch.cuda.synchronize()
        ref_lp = fresh.clone().requires_grad_(True)
        ref_out = api.ctc_loss(ref_lp, *args, **kw)  # eager work between replays
        ref_out.backward()
        torch.cuda.synchronize()
        assert torch.allclose(out.detach(), ref_out.detach(), rtol=1e-6, atol=0), k
        assert float((lp_static.grad.double() - ref_lp.grad.double()).abs().max()) <= 1e-6, k
        _say(f"  replay {k}: matches the eager forward + backward")


_FIRST_CALL_CAPTURED = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
from ctc_forward_backward_amd import api, workloads as W
b = W.make_workload("small")  # three utterance groups
dev = torch.device("cuda:0")
args = (b.cu_seqlens.to(dev), b.lengths.to(dev), b.targets.to(dev), b.target_lengths.to(dev))
kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction, max_target_length=int(b.targets.shape[1]))
lp = b.log_probs.to(dev).clone()
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):  # the process's first library call: no library streams exist yet
    losses, reduced, grad = api.packed_ctc_loss(lp, *args, **kw)
for k in range(2):
    rng = np.random.default_rng(200 + k)
    logits = rng.normal(0.0, 2.0, size=tuple(lp.shape))
    fresh = torch.from_numpy(logits).log_softmax(-1).to(lp.dtype).to(dev)
    lp.copy_(fresh)
    g.replay()
    torch.cuda.synchronize()
    el, er, eg = api.packed_ctc_loss(fresh, *args, **kw)
    torch.cuda.synchronize()
    assert torch.allclose(losses, el, rtol=1e-6, atol=0), k
    assert float((grad.double() - eg.double()).abs().max()) <= 1e-6, k
print("OK", flush=True)
"""


def test_graph_capture_as_first_call(api):
    """A call captured before the library has made its group streams runs as one group on the
    capturing stream; replays match eager calls.  Runs in a child process, so that no earlier call
    has made the streams."""
    import os
    import subprocess
    import sys

    _say("[gpu autograd] graph capture as a process's first call (child process)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED, root], capture_output=True, text=True, timeout=110)
    assert r.returncode == 0 and "OK" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])


def _replay_batches():
    """Metadata of the page's graph-replay scenario: four utterances in fixed row slots
    (cu_seqlens [0, 70, 77, 81, 81], D = 6, blank 5), a (4, 32) targets buffer; per replay new labels
    (junk past each length), target lengths and frame lengths."""
    rng = np.random.default_rng(19)
    out = []
    for tl, ln in (([4, 3, 2, 0], [70, 7, 4, 0]), ([32, 2, 1, 0], [70, 7, 4, 0]), ([0, 1, 2, 0], [66, 7, 0, 0]),
                   ([32, 3, 0, 0], [70, 5, 4, 0])):
        tg = rng.integers(0, 5, size=(4, 32))
        out.append((torch.tensor(tg, dtype=torch.int64), torch.tensor(tl, dtype=torch.int64),
                    torch.tensor(ln, dtype=torch.int64)))
    return out


def _replay_case():
    b = W.make_batch([70, 7, 4, 0], [[1, 2, 3, 4], [0, 1, 2], [3, 3], []], 6, seed=19, sigma=1.0, blank=5,
                     width=32)
    return b


def _oracle_for(oracle_mod, lp, cu, tg, tl, ln):
    return oracle_mod.ctc_packed(lp, cu, ln, tg, tl, blank=5, reduction="none")


@pytest.mark.parametrize("pipeline", ["streamed", "grouped"])
def test_graph_replay_new_metadata_fused(api, oracle_mod, pipeline):
    _say(f"[gpu autograd] graph replay with new targets / lengths, fused call, pipeline {pipeline}")
    api.set_pipeline(pipeline)
    try:
        b = _replay_case()
        dev = torch.device("cuda:0")
        lp = b.log_probs.to(dev)
        cu = b.cu_seqlens.to(dev)
        ln = b.lengths.to(dev)
        tg = b.targets.to(dev)
        tl = b.target_lengths.to(dev)
        kw = dict(blank=5, reduction="none", max_target_length=32)
        api.packed_ctc_loss(lp, cu, ln, tg, tl, **kw)  # eager first (the library's group streams)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            losses, _, grad = api.packed_ctc_loss(lp, cu, ln, tg, tl, **kw)
        for k, (ntg, ntl, nln) in enumerate(_replay_batches()):
            tg.copy_(ntg.to(dev))
            tl.copy_(ntl.to(dev))
            ln.copy_(nln.to(dev))
            graph.replay()
            torch.cuda.synchronize()
            assert api.last_call_status() == 0
            ref = _oracle_for(oracle_mod, b.log_probs, b.cu_seqlens, ntg, ntl, nln)
            _check_oracle(losses, grad, ref, torch.float32, f"replay {k} U={ntl.tolist()} T={nln.tolist()}")
            api.packed_ctc_loss(lp, cu, ln, tg, tl, **kw)  # eager work between replays
            torch.cuda.synchronize()
            assert float(losses[3]) == 0.0
    finally:
        api.set_pipeline("streamed")


def test_graph_replay_new_metadata_autograd(api, oracle_mod):
    _say("[gpu autograd] graph replay with new targets / lengths, autograd forward + backward")
    b = _replay_case()
    dev = torch.device("cuda:0")
    lp = b.log_probs.to(dev).clone().requires_grad_(True)
    cu = b.cu_seqlens.to(dev)
    ln = b.lengths.to(dev)
    tg = b.targets.to(dev)
    tl = b.target_lengths.to(dev)
    kw = dict(blank=5, reduction="none", max_target_length=32)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm-up outside the capture
        api.ctc_loss(lp, cu, ln, tg, tl, **kw).sum().backward()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    lp.grad = None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = api.ctc_loss(lp, cu, ln, tg, tl, **kw)
        out.sum().backward()
    for k, (ntg, ntl, nln) in enumerate(_replay_batches()):
        tg.copy_(ntg.to(dev))
        tl.copy_(ntl.to(dev))
        ln.copy_(nln.to(dev))
        graph.replay()
        torch.cuda.synchronize()
        ref = _oracle_for(oracle_mod, b.log_probs, b.cu_seqlens, ntg, ntl, nln)
        _check_oracle(out, lp.grad, ref, torch.float32, f"autograd replay {k} U={ntl.tolist()} T={nln.tolist()}")


@pytest.mark.parametrize("reduction", ["none", "mean"])
def test_float64_autograd_vs_oracle(api, oracle_mod, reduction):
    """float64 log probs through autograd: losses (float64) and the gradient with upstream weights,
    computed in float64, within 1e-10 of the oracle."""
    _say(f"[gpu autograd] float64 ctc_loss.backward, reduction {reduction}")
    rng = np.random.default_rng(41)
    lengths = [int(x) for x in rng.integers(1, 300, size=9)] + [0]
    tl = [int(rng.integers(0, max(1, T // 3) + 1)) for T in lengths]
    tl[-1] = 0
    targets = [[int(x) for x in rng.integers(1, 60, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, 60, seed=41, sigma=2.0, dtype="f64", reduction=reduction)
    lp = b.log_probs.to("cuda:0").requires_grad_(True)
    out = api.ctc_loss(lp, *_dev_args(b), blank=b.blank, reduction=reduction)
    assert out.dtype == torch.float64
    if reduction == "none":
        g = torch.linspace(-1.0, 1.0, b.B, dtype=torch.float64, device="cuda:0")
        out.backward(g)
        gs = g.cpu().numpy()
    else:
        out.backward(torch.tensor(0.75, dtype=torch.float64, device="cuda:0"))
        gs = np.full(b.B, 0.75)
    torch.cuda.synchronize()
    ref = oracle_mod.ctc_batch(b, reduction=reduction, grad_scale=gs)
    losses = out if reduction == "none" else torch.from_numpy(ref["loss"])
    _check_oracle(losses, lp.grad, ref, torch.float64, f"float64 autograd/{reduction}")
    if reduction != "none":
        np.testing.assert_allclose(float(out.detach().cpu()), ref["reduced"], rtol=1e-10, atol=0)
    assert lp.grad.dtype == torch.float64


@pytest.mark.parametrize("pipeline", ["streamed", "grouped"])
@pytest.mark.parametrize("zero_infinity", [False, True])
def test_split_edge_cases_vs_oracle(api, oracle_mod, pipeline, zero_infinity):
    # the split forward leaves the rows of utterances with a NaN input, without an alignment or with a
    # zero upstream weight to the backward: one frame short of U + repeats and exactly at it,
    # blank-id labels (blank 6), NaN at a label, at the blank and at a column no state reads
    _say(f"[gpu autograd] split forward / backward edge cases, {pipeline}, zero_infinity={zero_infinity}")
    import dataclasses

    cases = [([1, 1, 2], 3), ([1, 1, 2], 4), ([6, 6, 1], 3), ([6, 6, 1], 4), ([2, 4], 9), ([2, 4], 9),
             ([1, 1, 2], 3), ([5], 7), ([3], 40), ([], 12)]
    b = W.make_batch([T for _, T in cases], [t for t, _ in cases], 7, seed=41, sigma=1.5, blank=6,
                     zero_infinity=zero_infinity, reduction="none")
    lp = b.log_probs.clone()
    cu = [int(x) for x in b.cu_seqlens]
    lp[cu[4] + 4, 4] = float("nan")
    lp[cu[5] + 2, 6] = float("nan")
    lp[cu[6] + 1, 2] = float("nan")
    lp[cu[7] + 3, 0] = float("nan")
    b = dataclasses.replace(b, log_probs=lp)
    api.set_pipeline(pipeline)
    try:
        losses, _, state = api.packed_ctc_forward(lp.to("cuda:0"), *_dev_args(b), blank=6,
                                                  zero_infinity=zero_infinity, reduction="none")
        gs = np.linspace(-1.0, 1.0, b.B).astype(np.float32)
        gs[8] = 0.0
        grad = api.packed_ctc_backward(state, torch.from_numpy(gs), zero_infinity=zero_infinity, reduction="none")
        torch.cuda.synchronize()
    finally:
        api.set_pipeline("streamed")
    ref = oracle_mod.ctc_batch(b, reduction="none", grad_scale=gs.astype(np.float64))
    loss = losses.cpu().double().numpy()
    assert np.array_equal(np.isnan(loss), np.isnan(ref["loss"]))
    ok = ~np.isnan(ref["loss"])
    assert np.array_equal(np.isinf(loss[ok]), np.isinf(ref["loss"][ok]))
    fin = ok & ~np.isinf(ref["loss"])
    np.testing.assert_allclose(loss[fin], ref["loss"][fin], rtol=1e-4, atol=1e-5)
    g = grad.cpu().double().numpy()
    assert np.array_equal(np.isnan(g), np.isnan(ref["grad"]))
    m = ~np.isnan(ref["grad"])
    err = float(np.max(np.abs(g[m] - ref["grad"][m])))
    _say(f"  max |grad err| = {err:.3e}")
    assert err <= 1e-4
