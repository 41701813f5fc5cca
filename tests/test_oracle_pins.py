"""Pins of the float64 oracle against things other than itself.

- brute-force enumeration of every frame path (the definition of the CTC likelihood) on tiny inputs;
- closed forms: no labels, a tight single-path alignment, uniform log probabilities (path counting);
- an independent dense log-space HMM forward run on the CTC topology;
- torch.nn.functional.ctc_loss in float64 on a padded copy (the library the packed kernel page
  compares its kernel to), loss and gradient;
- central finite differences with respect to the logits;
- a hand-derived worked example stored under tests/golden/.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, hmm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lp(rng, T, D, sigma=1.0):
    z = rng.normal(0.0, sigma, size=(T, D))
    z = z - z.max(axis=1, keepdims=True)
    return z - np.log(np.exp(z).sum(axis=1, keepdims=True))


def _single(oracle_mod, lp, target, blank, zero_infinity=False, reduction="none"):
    T = lp.shape[0]
    tg = np.asarray(target, dtype=np.int64).reshape(1, -1) if len(target) else np.zeros((1, 0), dtype=np.int64)
    return oracle_mod.ctc_packed(lp, [0, T], [T], tg, [len(target)], blank=blank, zero_infinity=zero_infinity,
                                 reduction=reduction)


def _tiny_cases():
    rng = np.random.default_rng(1234)
    cases = []
    # hand-picked structures: repeats, a target equal to the blank id, U = 0, tight and infeasible lengths
    fixed = [
        (3, 3, [1, 1], 0),        # repeat needs a blank between: U + R = 3 = T (tight)
        (2, 3, [1, 1], 0),        # U + R = 3 > T: infeasible
        (4, 3, [2, 0, 2], 0),     # the blank id inside the targets is an ordinary label
        (4, 3, [0, 0], 0),        # repeated blank-id label
        (5, 4, [3, 1, 3], 3),     # blank = D - 1, targets hold the blank id
        (3, 2, [], 0),            # no labels
        (1, 3, [2], 0),           # single frame, single label
        (1, 3, [1, 2], 0),        # single frame, two labels: infeasible
        (6, 3, [1, 2, 1], 0),
        (6, 2, [1, 1, 1], 0),     # U + R = 5 <= 6
        (5, 4, [1, 2, 3], 2),     # blank in the middle of the class range
        (7, 2, [1], 0),
    ]
    for T, D, tgt, blank in fixed:
        cases.append((_lp(rng, T, D), tgt, blank))
    for _ in range(30):
        T = int(rng.integers(1, 7))
        D = int(rng.integers(2, 5))
        if D ** T > 5000:
            T = 5
        blank = int(rng.integers(0, D))
        U = int(rng.integers(0, 4))
        tgt = [int(x) for x in rng.integers(0, D, size=U)]
        cases.append((_lp(rng, T, D, sigma=1.5), tgt, blank))
    return cases


@pytest.mark.parametrize("idx", range(42))
def test_bruteforce_loss_and_gradient(oracle_mod, idx):
    lp, tgt, blank = _tiny_cases()[idx]
    # the state-path enumeration is the recursion's definition; without the blank id among the
    # targets it must equal the collapse definition, which is checked first
    nll_bf, post = brute.ctc_brute_states(lp, tgt, blank)
    if blank not in tgt:
        nll_c, post_c = brute.ctc_brute(lp, tgt, blank)
        if math.isinf(nll_c):
            assert math.isinf(nll_bf)
        else:
            np.testing.assert_allclose(nll_bf, nll_c, rtol=1e-12)
            np.testing.assert_allclose(post, post_c, atol=1e-12)
    for zi in (False, True):
        r = _single(oracle_mod, lp, tgt, blank, zero_infinity=zi)
        if math.isinf(nll_bf):
            assert math.isinf(r["nll"][0]) and r["nll"][0] > 0
            if zi:
                assert r["loss"][0] == 0.0
                assert np.all(r["grad"] == 0.0)
            else:
                assert math.isinf(r["loss"][0])
                assert np.all(np.isnan(r["grad"]))
        else:
            np.testing.assert_allclose(r["nll"][0], nll_bf, rtol=1e-12, atol=1e-12)
            expected = np.exp(lp) - post
            np.testing.assert_allclose(r["grad"], expected, rtol=0, atol=1e-12)


def test_bruteforce_covers_feasible_and_infeasible():
    kinds, with_blank = set(), 0
    for lp, tgt, blank in _tiny_cases():
        kinds.add(math.isinf(brute.ctc_brute_states(lp, tgt, blank)[0]))
        with_blank += blank in tgt
    assert kinds == {True, False}
    assert with_blank >= 3


def test_blank_id_target_differs_from_collapse_definition():
    # a target holding the blank id cannot come out of the collapse rule, yet the recursion scores it
    rng = np.random.default_rng(9)
    lp = _lp(rng, 4, 3)
    assert math.isinf(brute.ctc_brute(lp, [2, 0, 2], 0)[0])
    assert math.isfinite(brute.ctc_brute_states(lp, [2, 0, 2], 0)[0])


@pytest.mark.parametrize("T,D,blank", [(1, 3, 0), (5, 4, 2), (17, 6, 5), (40, 9, 0)])
def test_closed_form_no_labels(oracle_mod, T, D, blank):
    lp = _lp(np.random.default_rng(T), T, D)
    r = _single(oracle_mod, lp, [], blank)
    np.testing.assert_allclose(r["nll"][0], -lp[:, blank].sum(), rtol=1e-13)
    onehot = np.zeros_like(lp)
    onehot[:, blank] = 1.0
    np.testing.assert_allclose(r["grad"], np.exp(lp) - onehot, atol=1e-13)


@pytest.mark.parametrize("U,D", [(1, 3), (4, 6), (12, 20), (30, 31)])
def test_closed_form_tight_alignment(oracle_mod, U, D):
    # T = U and no two neighbouring labels equal: the only path emits one label per frame
    rng = np.random.default_rng(U)
    labels = list(rng.permutation(np.arange(1, D))[:U].astype(int))
    lp = _lp(rng, U, D)
    r = _single(oracle_mod, lp, labels, 0)
    np.testing.assert_allclose(r["nll"][0], -sum(lp[t, l] for t, l in enumerate(labels)), rtol=1e-13)
    onehot = np.zeros_like(lp)
    onehot[np.arange(U), labels] = 1.0
    np.testing.assert_allclose(r["grad"], np.exp(lp) - onehot, atol=1e-12)


@pytest.mark.parametrize("T,U", [(1, 1), (3, 1), (6, 2), (10, 3), (25, 7), (60, 20), (200, 50)])
def test_closed_form_uniform_path_count(oracle_mod, T, U):
    # every path has probability D**-T; the count of alignments of U distinct-neighbour labels is C(T+U, 2U)
    D = 7
    labels = [1 + (j % 3) for j in range(U)]  # 1,2,3,1,2,3,...: no neighbouring repeats
    lp = np.full((T, D), -math.log(D))
    r = _single(oracle_mod, lp, labels, 0)
    expected = T * math.log(D) - math.log(brute.count_alignments(T, U))
    np.testing.assert_allclose(r["nll"][0], expected, rtol=1e-12)


def test_path_count_formula_by_enumeration():
    # pins the counting formula itself on small sizes by enumerating paths
    D = 3
    for T in range(1, 7):
        for U in range(0, 3):
            labels = [1, 2][:U]
            n = sum(1 for p in __import__("itertools").product(range(D), repeat=T) if brute.collapse(p, 0) == labels)
            assert n == brute.count_alignments(T, U), (T, U)


@pytest.mark.parametrize("seed", range(12))
def test_dense_hmm_forward_agrees(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 60))
    D = int(rng.integers(2, 12))
    blank = int(rng.integers(0, D))
    U = int(rng.integers(0, max(1, T // 2) + 1))
    tgt = [int(x) for x in rng.integers(0, D, size=U)]
    if seed % 3 == 0 and U > 1:
        tgt[1] = tgt[0]  # a repeat
    lp = _lp(rng, T, D, sigma=2.0)
    r = _single(oracle_mod, lp, tgt, blank)
    ref = hmm.ctc_nll_via_hmm(lp, tgt, blank)
    if math.isinf(ref):
        assert math.isinf(r["nll"][0])
    else:
        np.testing.assert_allclose(r["nll"][0], ref, rtol=1e-12)


def _torch_reference(lp_flat, cu, lengths, targets, target_lengths, blank, zero_infinity):
    """Padded float64 torch.nn.functional.ctc_loss: per-utterance losses and d(sum loss)/d(lp) per packed row."""
    B = len(lengths)
    T_max = max([int(x) for x in lengths] + [1])
    D = lp_flat.shape[1]
    dense = torch.zeros(T_max, B, D, dtype=torch.float64)
    for b in range(B):
        r, T = int(cu[b]), int(lengths[b])
        dense[:T, b] = torch.from_numpy(lp_flat[r:r + T])
    dense.requires_grad_()
    loss = torch.nn.functional.ctc_loss(dense, torch.as_tensor(targets, dtype=torch.long),
                                        torch.as_tensor(lengths, dtype=torch.long),
                                        torch.as_tensor(target_lengths, dtype=torch.long), blank=blank,
                                        reduction="none", zero_infinity=zero_infinity)
    loss.sum().backward()
    g = np.zeros_like(lp_flat)
    for b in range(B):
        r, T = int(cu[b]), int(lengths[b])
        g[r:r + T] = dense.grad[:T, b].numpy()
    return loss.detach().numpy(), g


def _torch_cases():
    rng = np.random.default_rng(77)
    cases = []
    # the structures of the packed kernel page's tests (values are ours)
    cases.append(([8, 5, 2], [[1, 1, 2], [2, 0, 0], [0, 0, 0]], [3, 1, 0], 5, 4))      # small case, blank = D - 1
    cases.append(([9, 9, 7], [[1, 1, 2, 2], [4, 4, 1, 0], [2, 4, 2, 0]], [4, 3, 3], 5, 4))  # repeats and blank-id labels
    cases.append(([6, 3], [[], []], [0, 0], 3, 2))                                      # empty targets
    cases.append(([5, 0, 3], [[1, 2], [1, 0], [2, 0]], [2, 0, 1], 4, 3))               # a zero-length utterance
    for _ in range(6):
        B = int(rng.integers(1, 6))
        D = int(rng.integers(3, 40))
        blank = int(rng.integers(0, D))
        lengths = [int(x) for x in rng.integers(1, 120, size=B)]
        tl = [int(rng.integers(0, max(1, T // 3) + 1)) for T in lengths]
        W = max(tl + [1])
        tg = [[int(x) for x in rng.integers(0, D, size=W)] for _ in range(B)]
        cases.append((lengths, tg, tl, D, blank))
    return cases


@pytest.mark.parametrize("idx", range(10))
def test_against_torch_ctc_float64(oracle_mod, idx):
    lengths, tg, tl, D, blank = _torch_cases()[idx]
    rng = np.random.default_rng(idx)
    B = len(lengths)
    W = max([len(t) for t in tg] + [1])
    targets = np.zeros((B, W), dtype=np.int64)
    for b, t in enumerate(tg):
        targets[b, :len(t)] = t
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    lp = _lp(rng, int(cu[-1]), D, sigma=2.0)
    ref_loss, ref_grad = _torch_reference(lp, cu, lengths, targets, tl, blank, False)
    r = oracle_mod.ctc_packed(lp, cu, lengths, targets, tl, blank=blank)
    for b in range(B):
        if lengths[b] == 0:
            # a frameless utterance: 0 without labels, +inf with labels (torch agrees up to the sign of zero)
            assert r["nll"][b] == (0.0 if tl[b] == 0 else math.inf)
            continue
        np.testing.assert_allclose(r["nll"][b], ref_loss[b], rtol=1e-11)
    # torch's CPU gradient is off at the last frame when the last target equals the blank id
    # (test_last_target_blank_against_state_brute_force pins that case by enumeration instead)
    for b in range(B):
        rows = slice(int(cu[b]), int(cu[b]) + lengths[b])
        if tl[b] and targets[b, tl[b] - 1] == blank:
            continue
        np.testing.assert_allclose(r["grad"][rows], ref_grad[rows], atol=1e-11)


@pytest.mark.parametrize("tgt", [[1, 0], [0], [2, 1, 0], [0, 0]])
def test_last_target_blank_against_state_brute_force(oracle_mod, tgt):
    rng = np.random.default_rng(len(tgt))
    lp = _lp(rng, 5, 3)
    nll, post = brute.ctc_brute_states(lp, tgt, 0)
    r = _single(oracle_mod, lp, tgt, 0)
    np.testing.assert_allclose(r["nll"][0], nll, rtol=1e-12)
    np.testing.assert_allclose(r["grad"], np.exp(lp) - post, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_finite_differences_wrt_logits(oracle_mod, seed):
    rng = np.random.default_rng(500 + seed)
    lengths = [int(x) for x in rng.integers(3, 12, size=2)]
    D = int(rng.integers(3, 7))
    blank = int(rng.integers(0, D))
    tl = [int(rng.integers(1, max(2, T // 2))) for T in lengths]
    W = max(tl)
    targets = rng.integers(0, D, size=(2, W)).astype(np.int64)
    cu = np.array([0, lengths[0], lengths[0] + lengths[1]])
    z = rng.normal(size=(int(cu[-1]), D))
    scale = np.array([0.7, -1.3])

    def f(zz):
        lp = zz - zz.max(1, keepdims=True)
        lp = lp - np.log(np.exp(lp).sum(1, keepdims=True))
        r = oracle_mod.ctc_packed(lp, cu, lengths, targets, tl, blank=blank, want_grad=False)
        return float((r["nll"] * scale).sum())

    lp = z - z.max(1, keepdims=True)
    lp = lp - np.log(np.exp(lp).sum(1, keepdims=True))
    g = oracle_mod.ctc_packed(lp, cu, lengths, targets, tl, blank=blank, grad_scale=scale)["grad"]
    h = 1e-5
    fd = np.zeros_like(z)
    for i in range(z.shape[0]):
        for c in range(D):
            zp = z.copy(); zp[i, c] += h
            zm = z.copy(); zm[i, c] -= h
            fd[i, c] = (f(zp) - f(zm)) / (2 * h)
    np.testing.assert_allclose(g, fd, atol=2e-8)


def test_golden_hand_example(oracle_mod):
    with open(os.path.join(GOLDEN, "hand_two_frames.json")) as fh:
        gold = json.load(fh)
    lp = np.log(np.array(gold["probs"], dtype=np.float64))
    r = _single(oracle_mod, lp, gold["target"], gold["blank"])
    np.testing.assert_allclose(r["nll"][0], gold["nll"], rtol=1e-14)
    np.testing.assert_allclose(r["grad"], np.array(gold["grad"]), atol=1e-14)
