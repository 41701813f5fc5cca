"""HIP path vs the float64 oracle, element by element, through the C ABI.

Tolerances: losses within 1e-4 relative for float32 inputs, 2e-3 for bfloat16 / float16 inputs and
1e-10 for float64 inputs (computed in float64);
gradients within 1e-4 / 2e-3 absolute (the gradient is stored in the input dtype, so for bfloat16 /
float16 the rounding of the stored value is part of the budget).  Several results are correct where
the method sums repeated labels in any order; the comparison is tolerance-based throughout.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

from ctc_forward_backward_amd import workloads as W

pytestmark = pytest.mark.gpu

# float64 inputs are computed in float64: the precision the page's float64 path keeps (its test of
# that path compares at 1e-10)
TOL = {torch.float32: (1e-4, 1e-4), torch.float64: (1e-10, 1e-10), torch.bfloat16: (2e-3, 2e-3),
       torch.float16: (2e-3, 2e-3)}


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", params=["streamed", "grouped"])
def api(request):
    """The binding, with the loss + gradient calls of the module on one pipeline, then the other."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ctc_forward_backward_amd import api as _api

    _api._load()
    _api.set_pipeline(request.param)
    _say(f"pipeline: {request.param}")
    yield _api
    _api.set_pipeline("streamed")


def run_gpu(api, batch, *, reduction=None, grad_scale=None, need_grad=True, max_target_length=None,
            index_dtypes=None, cpu_targets=False):
    dev = torch.device("cuda:0")
    cu, ln, tg, tl = batch.cu_seqlens, batch.lengths, batch.targets, batch.target_lengths
    if index_dtypes is not None:
        cu, ln, tg, tl = (x.to(d) for x, d in zip((cu, ln, tg, tl), index_dtypes))
    if not cpu_targets:
        tg, tl = tg.to(dev), tl.to(dev)
    losses, reduced, grad = api.packed_ctc_loss(
        batch.log_probs.to(dev), cu.to(dev), ln.to(dev), tg, tl, blank=batch.blank,
        zero_infinity=batch.zero_infinity, reduction=batch.reduction if reduction is None else reduction,
        grad_scale=grad_scale, need_grad=need_grad, max_target_length=max_target_length)
    torch.cuda.synchronize()
    assert api.last_call_status() == 0, "a recursion block gave up waiting for its neighbour"
    return {
        "loss": losses.cpu().double().numpy(),
        "reduced": None if reduced is None else float(reduced.cpu()),
        "grad": None if grad is None else grad.cpu().double().numpy(),
        "grad_dtype": None if grad is None else grad.dtype,
    }


def compare(got, ref, dtype, label="", grad_tol=None):
    lrt, gat = TOL[dtype]
    gat = gat if grad_tol is None else grad_tol
    loss, rloss = got["loss"], ref["loss"]
    assert loss.shape == rloss.shape
    inf_ref = np.isinf(rloss)
    assert np.array_equal(np.isinf(loss), inf_ref), label
    fin = ~inf_ref
    np.testing.assert_allclose(loss[fin], rloss[fin], rtol=lrt, atol=0 if dtype == torch.float64 else 1e-5,
                               err_msg=label)
    if ref.get("reduced") is not None and got.get("reduced") is not None:
        # (the reduced value and the losses are stored as float32, float64 for float64 inputs)
        np.testing.assert_allclose(got["reduced"], ref["reduced"], rtol=max(lrt, 1e-7), atol=1e-6, err_msg=label)
    if got.get("grad") is not None:
        g, rg = got["grad"], ref["grad"]
        nan_ref = np.isnan(rg)
        assert np.array_equal(np.isnan(g), nan_ref), label
        ok = ~nan_ref
        err = np.abs(g[ok] - rg[ok])
        worst = float(err.max()) if err.size else 0.0
        _say(f"  {label}: max |grad err| = {worst:.3e} (tol {gat}), max loss rel err = "
             f"{float(np.max(np.abs(loss[fin] - rloss[fin]) / np.maximum(np.abs(rloss[fin]), 1e-30))) if fin.any() else 0:.3e}")
        assert worst <= gat, f"{label}: gradient error {worst} > {gat}"


@pytest.mark.parametrize("name", ["tiny", "small", "asr_bpe", "large_vocab", "char_level"])
def test_workload_full_size(api, oracle_mod, name):
    _say(f"[gpu parity] workload {name}")
    b = W.make_workload(name)
    got = run_gpu(api, b)
    ref = oracle_mod.ctc_batch(b)
    compare(got, ref, b.log_probs.dtype, name)
    assert got["grad_dtype"] == b.log_probs.dtype


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_dtypes_and_reductions(api, oracle_mod, dtype, reduction):
    _say(f"[gpu parity] dtype {dtype} reduction {reduction}")
    rng = np.random.default_rng(11)
    lengths = [int(x) for x in rng.integers(1, 300, size=9)] + [0]
    tl = [int(rng.integers(0, max(1, T // 3) + 1)) for T in lengths]
    tl[-1] = 0
    targets = [[int(x) for x in rng.integers(1, 200, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, 200, seed=5, sigma=2.5, dtype=dtype, reduction=reduction)
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), b.log_probs.dtype, f"{dtype}/{reduction}")


def test_grad_scale(api, oracle_mod):
    b = W.tiny()
    gs = torch.tensor([0.5, -2.0, 0.0, 3.0])
    for red in ("none", "mean"):
        got = run_gpu(api, b, reduction=red, grad_scale=gs)
        ref = oracle_mod.ctc_batch(b, reduction=red, grad_scale=gs.numpy())
        compare(got, ref, torch.float32, f"grad_scale/{red}")


def test_page_structures(api, oracle_mod):
    # the structures of the packed kernel page's tests, with our own seeded values
    cases = [
        ("small case", W.make_batch([8, 5, 2], [[1, 1, 2], [2], []], 5, seed=7, blank=4)),
        ("repeats and blank-id labels", W.make_batch([9, 9, 7], [[1, 1, 2, 2], [4, 4, 1], [2, 4, 2]], 5, seed=3,
                                                     blank=4)),
        ("empty targets", W.make_batch([6, 3], [[], []], 3, seed=5, blank=2)),
        ("production shape", W.make_batch([667, 401, 123, 50, 599, 300],
                                          [list(np.random.default_rng(13).integers(0, 1026, size=T // 6))
                                           for T in [667, 401, 123, 50, 599, 300]], 1027, seed=13, blank=1026,
                                          reduction="mean")),
        ("last target is the blank id", W.make_batch([12, 7], [[3, 1, 0], [0]], 4, seed=2, blank=0)),
    ]
    for label, b in cases:
        _say(f"[gpu parity] {label}")
        compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.float32, label)


@pytest.mark.parametrize("zero_infinity", [False, True])
def test_zero_length_and_impossible(api, oracle_mod, zero_infinity):
    _say(f"[gpu parity] zero-length / impossible, zero_infinity={zero_infinity}")
    b = W.make_batch([5, 0, 3, 1, 6], [[1, 2], [1], [2], [1, 1], [2, 2, 2]], 4, seed=11, blank=3,
                     zero_infinity=zero_infinity)
    got = run_gpu(api, b)
    ref = oracle_mod.ctc_batch(b)
    compare(got, ref, torch.float32, "zero-length/impossible")
    assert got["loss"][1] == (0.0 if zero_infinity else math.inf)
    assert got["loss"][3] == (0.0 if zero_infinity else math.inf)  # T=1 with a repeat: no alignment
    if zero_infinity:
        assert np.all(got["grad"][8:9] == 0.0)


def _boundary_batch(zero_infinity, reduction):
    """Utterances one frame short of the fewest frames their labels need (U + repeats) beside ones
    with exactly that many; equal neighbours, blank-id labels (blank 6), a 300-label target over
    several state blocks; NaN log probs at the blank, at a label and at another column, with and
    without an alignment."""
    rng = np.random.default_rng(31)
    long_t = [int(x) for x in rng.integers(1, 4, size=300)]
    need = len(long_t) + sum(1 for i in range(1, len(long_t)) if long_t[i] == long_t[i - 1])
    cases = [([1, 1, 2], 3), ([1, 1, 2], 4), ([3, 3, 3], 4), ([3, 3, 3], 5), ([6, 6, 1], 3), ([6, 6, 1], 4),
             (long_t, need - 1), (long_t, need), ([2, 4], 9), ([2, 4], 9), ([1, 1, 2], 3), ([5], 7)]
    targets = [t for t, _ in cases]
    lengths = [T for _, T in cases]
    b = W.make_batch(lengths, targets, 7, seed=32, sigma=1.5, blank=6, zero_infinity=zero_infinity,
                     reduction=reduction)
    lp = b.log_probs.clone()
    cu = [int(x) for x in b.cu_seqlens]
    lp[cu[8] + 4, 4] = float("nan")   # a label column, alignment exists
    lp[cu[9] + 2, 6] = float("nan")   # the blank column, alignment exists
    lp[cu[10] + 1, 2] = float("nan")  # a label column, no alignment
    lp[cu[11] + 3, 0] = float("nan")  # a column no state reads
    return dataclasses.replace(b, log_probs=lp)


@pytest.mark.parametrize("zero_infinity", [False, True])
def test_no_alignment_boundary_and_nan_inputs(api, oracle_mod, zero_infinity):
    # an utterance with fewer frames than U + repeats runs no recursion (its loss is known to be
    # +inf, or NaN with a NaN at a column the recursion reads); one with exactly that many aligns
    _say(f"[gpu parity] no-alignment boundary and NaN inputs, zero_infinity={zero_infinity}")
    for reduction in ("none", "mean"):
        b = _boundary_batch(zero_infinity, reduction)
        ref = oracle_mod.ctc_batch(b)
        got = run_gpu(api, b)
        compare(got, ref, torch.float32, f"boundary/{reduction}")
        nll = ref["nll"]
        assert np.isinf(nll[[0, 2, 4, 6]]).all() and np.isfinite(nll[[1, 3, 5, 7]]).all()
        assert np.isnan(got["loss"][[8, 9, 10]]).all() and np.isfinite(got["loss"][11])
    # and with alpha kept every 8th step (the grouped pipeline's checkpointed arrangement)
    b = _boundary_batch(zero_infinity, "none")
    dev = torch.device("cuda:0")
    losses, _, grad = api.packed_ctc_loss(*(x.to(dev) for x in (b.log_probs, b.cu_seqlens, b.lengths, b.targets,
                                                                b.target_lengths)),
                                          blank=6, zero_infinity=zero_infinity, reduction="none",
                                          checkpoint_interval=8)
    torch.cuda.synchronize()
    got = {"loss": losses.cpu().double().numpy(), "grad": grad.cpu().double().numpy()}
    compare(got, oracle_mod.ctc_batch(b), torch.float32, "boundary K=8")


def test_over_allocated_targets_fillers_and_gaps(api, oracle_mod):
    _say("[gpu parity] over-allocated targets, fillers, gaps")
    tight = W.make_batch([9, 7, 4], [[1, 2, 3, 1], [2, 2, 4], [4, 1]], 6, seed=17, blank=5)
    wide = W.make_batch([9, 7, 4, 0, 0], [[1, 2, 3, 1], [2, 2, 4], [4, 1], [], []], 6, seed=17, blank=5, width=32,
                        gaps=[2, 3, 0, 1, 0], T_total=30)
    a = run_gpu(api, tight)
    g = run_gpu(api, wide)
    compare(g, oracle_mod.ctc_batch(wide), torch.float32, "wide")
    assert np.all(g["loss"][3:] == 0.0)
    owned = np.zeros(30, dtype=bool)
    for b in range(3):
        r0 = int(wide.cu_seqlens[b])
        owned[r0:r0 + int(wide.lengths[b])] = True
    assert np.all(g["grad"][~owned] == 0.0)
    # same utterances, same values -> same losses whether the width is 4 or 32
    tight2 = W.make_batch([9, 7, 4], [[1, 2, 3, 1], [2, 2, 4], [4, 1]], 6, seed=17, blank=5, width=32)
    tight2.log_probs = tight.log_probs.clone()  # the junk draw shifts the generator; reuse the values
    np.testing.assert_allclose(run_gpu(api, tight2)["loss"], a["loss"], rtol=1e-6)


@pytest.mark.parametrize("dt", [(torch.int32,) * 4, (torch.int64,) * 4, (torch.int32, torch.int64, torch.int32,
                                                                          torch.int64)])
def test_index_dtypes_and_cpu_targets(api, oracle_mod, dt):
    b = W.tiny()
    ref = oracle_mod.ctc_batch(b)
    compare(run_gpu(api, b, index_dtypes=dt), ref, torch.float32, f"index {dt}")
    compare(run_gpu(api, b, index_dtypes=dt, cpu_targets=True), ref, torch.float32, "cpu targets")


def test_long_targets_multiple_pairs_per_lane(api, oracle_mod):
    # U up to 3000 -> more than 1024 state pairs per utterance, several pairs per lane
    _say("[gpu parity] long targets")
    rng = np.random.default_rng(8)
    lengths = [6500, 3100, 40]
    tl = [3000, 1500, 10]
    targets = [[int(x) for x in rng.integers(1, 64, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, 64, seed=8, sigma=2.0, reduction="mean")
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.float32, "long targets")


@pytest.mark.parametrize("B", [2048, 7200])
def test_many_short_utterances(api, oracle_mod, B):
    # 2048: the streamed pipeline's largest batch (4096 recursion segments, far more than compute
    # units, so segments wait for free workgroups; the schedule's prefix sums and band queue at full
    # size).  7200: more utterances than the schedule sorts (one group, utterance order)
    _say(f"[gpu parity] {B} short utterances")
    rng = np.random.default_rng(B)
    lengths = [int(x) for x in rng.integers(1, 41, size=B)]
    tl = [int(min(x, max(t // 2, 0))) for x, t in zip(rng.integers(0, 11, size=B), lengths)]
    targets = [[int(v) for v in rng.integers(1, 16, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, 16, seed=B, sigma=1.0, reduction="mean")
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.float32, f"B={B}")


def test_concurrent_calls_on_two_streams(api, oracle_mod):
    # two calls in flight at once, each on its own stream with its own workspace: on the streamed
    # pipeline two persistent launches share the compute units, on the grouped one the library's
    # group streams
    _say("[gpu parity] two calls on two streams")
    dev = torch.device("cuda:0")
    batches = [W.make_workload("small"), W.make_workload("char_level")]
    ins = [(b.log_probs.to(dev), b.cu_seqlens.to(dev), b.lengths.to(dev), b.targets.to(dev), b.target_lengths.to(dev))
           for b in batches]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for b, x, st in zip(batches, ins, streams):
        with torch.cuda.stream(st):
            outs.append(api.packed_ctc_loss(*x, blank=b.blank, zero_infinity=b.zero_infinity, reduction=b.reduction,
                                            max_target_length=int(b.target_lengths.max())))
    torch.cuda.synchronize()
    for b, (losses, reduced, grad) in zip(batches, outs):
        got = {"loss": losses.cpu().double().numpy(), "reduced": float(reduced.cpu()),
               "grad": grad.cpu().double().numpy()}
        compare(got, oracle_mod.ctc_batch(b), torch.float32, f"{b.name} beside another call")


def test_utterance_beyond_band_buckets(api, oracle_mod):
    # one utterance of 70000 frames: the streamed pipeline's band queue takes its exact-count order
    # (the bucketed order covers up to 65535 frames); a short one beside it
    _say("[gpu parity] 70000-frame utterance")
    rng = np.random.default_rng(9)
    lengths = [70000, 300]
    tl = [60, 20]
    targets = [[int(x) for x in rng.integers(1, 8, size=u)] for u in tl]
    # and one without alignment (5 frames, 4 equal labels need 7), whose bands go first
    lengths.append(5)
    targets.append([3, 3, 3, 3])
    b = W.make_batch(lengths, targets, 8, seed=9, sigma=1.0, reduction="sum", zero_infinity=True)
    ref = oracle_mod.ctc_batch(b)
    got = run_gpu(api, b)
    current = api.pipeline()
    api.set_pipeline("grouped" if current == "streamed" else "streamed")
    try:
        other = run_gpu(api, b)
    finally:
        api.set_pipeline(current)
    # the two pipelines share the recursions: their posteriors agree to float32 rounding
    assert float(np.max(np.abs(got["grad"] - other["grad"]))) <= 1e-5
    np.testing.assert_allclose(got["loss"], ref["loss"], rtol=1e-4)
    # the recursions keep an integer offset per state pair, so float32 rounding does not accumulate
    # with the number of frames (with one offset per 64-pair block this case drifted to 8e-4)
    err = float(np.max(np.abs(got["grad"] - ref["grad"])))
    _say(f"  T=70000: max |grad err| = {err:.3e} (bar 1e-4)")
    assert err <= 1e-4


def test_large_vocabulary_lds_accumulator(api, oracle_mod):
    _say("[gpu parity] D = 30000")
    rng = np.random.default_rng(9)
    lengths = [200, 120]
    targets = [[int(x) for x in rng.integers(0, 29999, size=u)] for u in (40, 25)]
    b = W.make_batch(lengths, targets, 30000, seed=9, sigma=3.0, dtype="bf16", blank=29999, reduction="sum")
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.bfloat16, "D=30000")


@pytest.mark.parametrize("dtype,D", [("f16", 4096), ("f32", 1024)])
def test_wide_rows_class_and_label_order(api, oracle_mod, dtype, D):
    # rows of 4 KB or more: the streamed gather reads utterances of up to 512 labels in class order
    # and longer ones in label order; both kinds, a label-free utterance and an unowned row between
    # utterances, next to each other so that waves pass from one kind to the other
    _say(f"[gpu parity] wide rows, both gather orders ({dtype}, D = {D})")
    rng = np.random.default_rng(21)
    lengths = [1500, 640, 7, 900, 3100]
    tl = [700, 300, 0, 511, 1500]  # (the last: more classes than a wave's LDS list holds)
    targets = [[int(x) for x in rng.integers(1, D, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, D, seed=21, sigma=3.0, dtype=dtype, reduction="sum", gaps=[0, 0, 1, 0, 0])
    ref = oracle_mod.ctc_batch(b)
    got = run_gpu(api, b)
    compare(got, ref, torch.float16 if dtype == "f16" else torch.float32, f"wide rows {dtype}")


def test_loss_only_and_explicit_bound(api, oracle_mod):
    b = W.small()
    ref = oracle_mod.ctc_batch(b, want_grad=False)
    got = run_gpu(api, b, need_grad=False, max_target_length=int(b.target_lengths.max()))
    assert got["grad"] is None
    compare(got, ref, torch.float32, "loss only")
    # a looser caller bound gives the same result
    got2 = run_gpu(api, b, need_grad=False, max_target_length=int(b.targets.shape[1]))
    np.testing.assert_allclose(got2["loss"], got["loss"], rtol=1e-6)


def test_host_read_errors(api):
    b = W.tiny()
    dev = torch.device("cuda:0")
    args = (b.log_probs.to(dev), b.cu_seqlens.to(dev), b.lengths.to(dev), b.targets.to(dev))
    with pytest.raises(ValueError, match="negative"):
        api.packed_ctc_loss(*args, torch.tensor([3, -1, 2, 2], device=dev), blank=0)
    with pytest.raises(ValueError, match="targets row"):
        api.packed_ctc_loss(*args, b.target_lengths.to(dev) + 100, blank=0)
    with pytest.raises(TypeError, match="float32"):  # float64 is accepted (its own path); integers are not
        api.packed_ctc_loss(b.log_probs.to(torch.int32).to(dev), *args[1:], b.target_lengths.to(dev), blank=0)
    with pytest.raises(ValueError, match="blank"):
        api.packed_ctc_loss(*args, b.target_lengths.to(dev), blank=16)


def test_reduce_entry_point(api):
    dev = torch.device("cuda:0")
    losses = torch.tensor([1.0, 4.0, 9.0], device=dev)
    tl = torch.tensor([0, 2, 3], device=dev)
    assert abs(float(api.packed_ctc_reduce(losses, tl, "sum")) - 14.0) < 1e-6
    assert abs(float(api.packed_ctc_reduce(losses, tl, "mean")) - (1.0 + 2.0 + 3.0) / 3) < 1e-6
    empty = api.packed_ctc_reduce(torch.zeros(0, device=dev), torch.zeros(0, dtype=torch.long, device=dev), "mean")
    assert math.isnan(float(empty))


def test_empty_batch(api):
    dev = torch.device("cuda:0")
    lp = torch.randn(7, 4, device=dev).log_softmax(-1)
    losses, red, grad = api.packed_ctc_loss(lp, torch.zeros(1, dtype=torch.int32, device=dev),
                                            torch.zeros(0, dtype=torch.long, device=dev),
                                            torch.zeros(0, 3, dtype=torch.long, device=dev),
                                            torch.zeros(0, dtype=torch.long, device=dev), blank=0, reduction="sum")
    torch.cuda.synchronize()
    assert losses.numel() == 0 and float(red) == 0.0
    assert torch.all(grad == 0)


def test_repeatable_within_tolerance(api):
    b = W.asr_bpe()
    a = run_gpu(api, b)
    c = run_gpu(api, b)
    np.testing.assert_allclose(a["loss"], c["loss"], rtol=1e-6)
    np.testing.assert_allclose(np.nan_to_num(a["grad"]), np.nan_to_num(c["grad"]), atol=2e-3)


@pytest.mark.parametrize("reduction", ["none", "mean"])
def test_float64_inputs(api, oracle_mod, reduction):
    """float64 log probs computed in float64 throughout, gradient written as float64: 1e-10 against the
    oracle; several tiles of a 1025-class row and a ragged tail."""
    _say(f"[gpu parity] float64 inputs, reduction {reduction}")
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 400, size=11)] + [0, 3]
    tl = [int(rng.integers(0, max(1, T // 3) + 1)) for T in lengths]
    tl[-2] = 0
    targets = [[int(x) for x in rng.integers(1, 1025, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, 1025, seed=9, sigma=3.0, dtype="f64", reduction=reduction)
    got = run_gpu(api, b)
    assert got["grad_dtype"] == torch.float64
    compare(got, oracle_mod.ctc_batch(b), torch.float64, f"f64/{reduction}")


# float64 gradients agree with the oracle to 1e-10 while the recursion's log values stay below about
# 2e4 in size; past that the two sides' own rounding over thousands of frames sets the agreement (the
# 8260-frame case, loss 3.95e4: 1.04e-10, the same with the kernels before and after their rewrite)
@pytest.mark.parametrize("U,D,gtol", [(100, 2500, None), (255, 64, None), (256, 64, None), (511, 64, None),
                                      (600, 64, None), (2100, 64, None), (4100, 64, 2e-10)])
def test_float64_workgroup_shapes(api, oracle_mod, U, D, gtol):
    """float64 at each workgroup shape the longest target selects (512 threads up to 511 labels, then
    1024 threads of 4, 8 or 16 states) and on both sides of each boundary, beside a short utterance;
    D = 2500 runs the gradient row past the columns a thread keeps in registers."""
    _say(f"[gpu parity] float64 workgroup shape: U = {U}, D = {D}")
    rng = np.random.default_rng(40 + U)
    targets = [[int(x) for x in rng.integers(1, D, size=U)], [int(x) for x in rng.integers(1, D, size=5)]]
    b = W.make_batch([2 * U + 60, 23], targets, D, seed=41 + U, sigma=3.0, dtype="f64", reduction="none")
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.float64, f"f64 U={U} D={D}", grad_tol=gtol)


def test_maximum_sizes(api, oracle_mod):
    """The library's limits: a target of 8191 labels (16383 states: 128 state blocks, 32 segments per
    recursion) over 8800 frames, and D = 32768 classes with the blank at the last class."""
    lim_u, lim_d = api.limits()
    _say(f"[gpu parity] maximum sizes: U = {lim_u}, D = {lim_d}")
    rng = np.random.default_rng(12)
    targets = [[int(x) for x in rng.integers(1, 64, size=lim_u)], [int(x) for x in rng.integers(1, 64, size=7)]]
    b = W.make_batch([8800, 30], targets, 64, seed=12, sigma=1.5, reduction="none")
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.float32, f"U={lim_u}")
    targets = [[int(x) for x in rng.integers(0, lim_d - 1, size=u)] for u in (30, 12, 0)]
    b = W.make_batch([90, 41, 5], targets, lim_d, seed=13, sigma=3.0, dtype="bf16", blank=lim_d - 1,
                     reduction="mean")
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.bfloat16, f"D={lim_d}")


def test_wait_give_up_poisons_the_call(api, oracle_mod):
    """Every wait of one wave on another is bounded in wall-clock time.  With the bound set to 0 from
    the host, the waits that are not met at once give up; every kernel still ends, the call's losses
    and reduced value come back NaN and the workspace status is non-zero.  A call after the bound is
    restored is healthy and matches the oracle."""
    _say("[gpu parity] bounded waits forced to give up (wait limit 0)")
    rng = np.random.default_rng(23)
    lengths = [1800, 900, 300]
    tl = [600, 250, 40]  # 10, 4 and 1 state blocks: a chain of three segments, one of one segment
    targets = [[int(x) for x in rng.integers(1, 40, size=u)] for u in tl]
    b = W.make_batch(lengths, targets, 40, seed=23, sigma=1.5, reduction="sum")
    dev = torch.device("cuda:0")
    old = api.wait_limit()
    api.set_wait_limit(0)
    try:
        losses, reduced, grad = api.packed_ctc_loss(b.log_probs.to(dev), b.cu_seqlens.to(dev), b.lengths.to(dev),
                                                    b.targets.to(dev), b.target_lengths.to(dev), blank=b.blank,
                                                    reduction="sum", max_target_length=max(tl))
        torch.cuda.synchronize()
        status = api.last_call_status()
    finally:
        api.set_wait_limit(old)
    _say(f"  status {status}, losses {losses.cpu().tolist()}")
    assert status != 0
    assert bool(torch.isnan(losses).all()) and bool(torch.isnan(reduced))
    compare(run_gpu(api, b), oracle_mod.ctc_batch(b), torch.float32, "after the bound is restored")
