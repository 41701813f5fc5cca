"""Alpha checkpointing (checkpoint_interval K) on the GPU, through the C ABI, against the oracle.

With K > 1 the alpha recursion keeps every K-th step of each utterance and the rows of each K-step
interval recompute alpha from the kept step (the page's Triton file keeps every alpha row,
`_alpha_kernel` / `_beta_grad_kernel`; the interval only changes what is stored, not what is
computed).  Every workload is checked at K = 1, 8 and 32, on the fused call and on the split
forward / backward, at the parity bars (losses 1e-4 / 2e-3 relative, gradients 1e-4 / 2e-3
absolute for float32 / 16-bit inputs); K > 1 also agrees with K = 1.  The workspace each K needs is
printed.
"""

import numpy as np
import pytest
import torch

from ctc_forward_backward_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-4, 1e-4), torch.bfloat16: (2e-3, 2e-3), torch.float16: (2e-3, 2e-3)}


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ctc_forward_backward_amd import api as _api

    _api._load()
    return _api


def _dev(b):
    d = torch.device("cuda:0")
    return (b.log_probs.to(d), b.cu_seqlens.to(d), b.lengths.to(d), b.targets.to(d), b.target_lengths.to(d))


def _check(losses, grad, ref, dtype, label):
    lrt, gat = TOL[dtype]
    loss = losses.detach().cpu().double().numpy()
    rloss = ref["loss"]
    assert np.array_equal(np.isinf(loss), np.isinf(rloss)), label
    fin = ~np.isinf(rloss)
    np.testing.assert_allclose(loss[fin], rloss[fin], rtol=lrt, atol=1e-5, err_msg=label)
    g = grad.detach().cpu().double().numpy()
    rg = ref["grad"]
    nan_ref = np.isnan(rg)
    assert np.array_equal(np.isnan(g), nan_ref), label
    err = np.abs(g - rg)[~nan_ref]
    worst = float(err.max()) if err.size else 0.0
    _say(f"  {label}: max |grad err| = {worst:.3e} (tol {gat})")
    assert worst <= gat, f"{label}: gradient error {worst} > {gat}"
    return g


@pytest.mark.parametrize("name", ["tiny", "small", "asr_bpe", "large_vocab", "char_level"])
def test_workloads_at_checkpoint_intervals(api, oracle_mod, name):
    _say(f"[gpu checkpoint] workload {name}")
    b = W.make_workload(name)
    args = _dev(b)
    Umax = int(b.target_lengths.max())
    ref = oracle_mod.ctc_batch(b)
    grads = {}
    for K in (1, 8, 32):
        ws = api.packed_ctc_workspace_size(b.T_total, b.D, b.B, Umax, K)
        losses, _, grad = api.packed_ctc_loss(*args, blank=b.blank, zero_infinity=b.zero_infinity,
                                              reduction=b.reduction, max_target_length=Umax, checkpoint_interval=K)
        torch.cuda.synchronize()
        assert api.last_call_status() == 0
        _say(f"  K={K}: workspace {ws / 1e6:.1f} MB")
        grads[K] = _check(losses, grad, ref, b.log_probs.dtype, f"{name} fused K={K}")
        # the split entry points with the same interval (the autograd boundary)
        l2, _, state = api.packed_ctc_forward(*args, blank=b.blank, zero_infinity=b.zero_infinity,
                                              reduction=b.reduction, max_target_length=Umax, checkpoint_interval=K)
        g2 = api.packed_ctc_backward(state, zero_infinity=b.zero_infinity)
        torch.cuda.synchronize()
        _check(l2, g2, ref, b.log_probs.dtype, f"{name} split K={K}")
    # the kept steps change only the rounding of the recomputed alpha: both results lie within the bar
    # of the oracle, so within twice the bar of each other (for 16-bit gradients a value near a
    # rounding boundary can land one stored ulp apart)
    for K in (8, 32):
        d = np.nan_to_num(grads[K]) - np.nan_to_num(grads[1])
        assert float(np.abs(d).max()) <= 2 * TOL[b.log_probs.dtype][1]


def test_ragged_intervals_and_edge_cases(api, oracle_mod):
    # lengths around multiples of the interval, single frames, empty targets, a zero-length utterance,
    # an infeasible one (no zero_infinity: its rows are NaN), repeats and blank-id labels
    _say("[gpu checkpoint] ragged intervals and edge cases")
    lengths = [1, 7, 8, 9, 31, 32, 33, 65, 0, 3, 40]
    rng = np.random.default_rng(5)
    targets = []
    for T in lengths:
        u = int(rng.integers(0, max(1, T // 3) + 1))
        targets.append([int(x) for x in rng.integers(0, 6, size=u)])
    targets[3] = []
    targets[8] = [1, 2]       # T = 0 with labels: infinite loss, no rows
    targets[9] = [2, 2, 2]    # T = 3 with two repeats: no alignment
    b = W.make_batch(lengths, targets, 7, seed=6, sigma=1.5, blank=6, reduction="none")
    args = _dev(b)
    ref = oracle_mod.ctc_batch(b)
    for K in (2, 8, 32):
        losses, _, grad = api.packed_ctc_loss(*args, blank=6, reduction="none", checkpoint_interval=K)
        torch.cuda.synchronize()
        _check(losses, grad, ref, torch.float32, f"edge cases K={K}")


def test_long_targets_at_the_checkpoint_limit(api, oracle_mod):
    # 1023 labels: 16 state blocks, the most a checkpointed utterance takes, beside a short one
    _say("[gpu checkpoint] 1023 labels")
    rng = np.random.default_rng(17)
    targets = [[int(x) for x in rng.integers(1, 50, size=1023)], [int(x) for x in rng.integers(1, 50, size=30)]]
    b = W.make_batch([2600, 200], targets, 50, seed=17, sigma=1.5, reduction="mean")
    args = _dev(b)
    ref = oracle_mod.ctc_batch(b)
    losses, _, grad = api.packed_ctc_loss(*args, blank=0, reduction="mean", checkpoint_interval=16)
    torch.cuda.synchronize()
    _check(losses, grad, ref, torch.float32, "U=1023 K=16")
    with pytest.raises(ValueError, match="checkpointing"):
        t2 = [[int(x) for x in rng.integers(1, 50, size=1024)]]
        b2 = W.make_batch([2100], t2, 50, seed=18)
        api.packed_ctc_loss(*_dev(b2), blank=0, checkpoint_interval=16)


def test_block_classes_in_one_batch(api, oracle_mod):
    # targets on both sides of each boundary of the 1-4 / 5-8 / 9-16 state-block classes (a target of
    # U labels takes (U + 64) // 64 blocks), in one batch and in a mixed order, at K = 8 and 4
    _say("[gpu checkpoint] every block class in one batch")
    rng = np.random.default_rng(23)
    ulist = [255, 0, 511, 256, 1023, 512, 40, 700, 191]
    lengths = [2 * u + 40 for u in ulist]
    targets = [[int(x) for x in rng.integers(1, 60, size=u)] for u in ulist]
    b = W.make_batch(lengths, targets, 60, seed=23, sigma=1.5, reduction="none")
    args = _dev(b)
    ref = oracle_mod.ctc_batch(b)
    for K in (8, 4):
        losses, _, grad = api.packed_ctc_loss(*args, blank=0, reduction="none", checkpoint_interval=K)
        torch.cuda.synchronize()
        _check(losses, grad, ref, torch.float32, f"block classes K={K}")


def test_graph_capture_checkpointed_groups(api):
    # a checkpointed call on a batch large enough to run in length-sorted groups on the library's
    # streams, captured in a graph after an eager call; each replay with fresh log probs (and eager
    # calls between replays) matches the eager call
    _say("[gpu checkpoint] graph capture of a grouped checkpointed call")
    b = W.make_workload("asr_bpe")
    dev = torch.device("cuda:0")
    args = _dev(b)[1:]
    kw = dict(blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction,
              max_target_length=int(b.targets.shape[1]), checkpoint_interval=8)
    lp_static = b.log_probs.to(dev).clone()
    api.packed_ctc_loss(lp_static, *args, **kw)  # eager first: the library's group streams exist
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        losses, reduced, grad = api.packed_ctc_loss(lp_static, *args, **kw)
    gen = torch.Generator(device=dev)
    for k in range(3):
        gen.manual_seed(200 + k)
        x = torch.randn(tuple(lp_static.shape), device=dev, generator=gen) * 2.0
        fresh = torch.log_softmax(x, dim=1).to(lp_static.dtype)
        lp_static.copy_(fresh)
        graph.replay()
        torch.cuda.synchronize()
        el, er, eg = api.packed_ctc_loss(fresh, *args, **kw)  # eager work between replays
        torch.cuda.synchronize()
        assert api.last_call_status() == 0
        fin = torch.isfinite(el)
        assert torch.equal(torch.isfinite(losses), fin), k
        assert torch.allclose(losses[fin], el[fin], rtol=1e-6, atol=0), k
        assert torch.allclose(reduced, er, rtol=1e-6, atol=0, equal_nan=True), k
        assert torch.equal(torch.isnan(grad), torch.isnan(eg)), k
        assert float((grad.double() - eg.double()).nan_to_num().abs().max()) <= 1e-6, k
        _say(f"  replay {k}: matches the eager call")
