"""Invariants of the float64 oracle, its reductions, and planted mistakes that the pins must catch.

Invariants (each holds for the exact method, so they pin the oracle at any size):
- the state posteriors of every frame of a feasible utterance sum to 1, and the two ways of forming
  them (exp(alpha + beta - lp + nll) and the per-frame softmax over states) agree;
- each gradient row sums to weight * (sum exp(lp) - 1), i.e. ~0 for normalised log probabilities;
- losses of normalised log probabilities are >= 0;
- an infeasible target gives +inf, and 0 with an all-zero gradient under zero_infinity;
- results do not depend on the order of the utterances, on an over-allocated targets buffer with
  junk past each length, on zero-length filler utterances, or on unowned (gap) rows, which get 0.
"""

import math
import os
import subprocess

import numpy as np
import pytest
import torch

from ctc_forward_backward_amd import workloads as W
from oracle import brute, oracle


def _lp(rng, T, D, sigma=1.0):
    z = rng.normal(0.0, sigma, size=(T, D))
    z = z - z.max(axis=1, keepdims=True)
    return z - np.log(np.exp(z).sum(axis=1, keepdims=True))


@pytest.mark.parametrize("seed", range(6))
def test_posteriors_sum_to_one(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(5, 300))
    D = int(rng.integers(3, 50))
    U = int(rng.integers(1, max(2, T // 3)))
    tgt = rng.integers(1, D, size=U)
    if U > 2:
        tgt[2] = tgt[1]
    lp = _lp(rng, T, D, sigma=3.0)
    r = oracle_mod.posteriors(lp, tgt, 0)
    assert math.isfinite(r["nll"])
    np.testing.assert_allclose(r["gamma"].sum(axis=1), 1.0, atol=1e-11)
    np.testing.assert_allclose(r["gamma"], r["gamma_norm"], atol=1e-11)


def test_gradient_rows_sum_to_zero_and_losses_nonnegative(oracle_mod):
    b = W.small()
    r = oracle_mod.ctc_batch(b, reduction="sum")
    lp = b.log_probs.double().numpy()
    row_sums = r["grad"].sum(axis=1)
    np.testing.assert_allclose(row_sums, np.exp(lp).sum(axis=1) - 1.0, atol=1e-11)
    assert np.all(r["loss"] >= 0)


def test_infeasible_and_zero_infinity(oracle_mod):
    rng = np.random.default_rng(3)
    lengths = [4, 6]
    lp = _lp(rng, 10, 5)
    targets = np.array([[1, 1, 2, 2], [1, 2, 3, 4]])  # utterance 0: U + R = 6 > 4
    tl = [4, 4]
    cu = [0, 4, 10]
    a = oracle_mod.ctc_packed(lp, cu, lengths, targets, tl, blank=0)
    z = oracle_mod.ctc_packed(lp, cu, lengths, targets, tl, blank=0, zero_infinity=True)
    assert math.isinf(a["loss"][0]) and a["loss"][0] > 0
    assert np.all(np.isnan(a["grad"][0:4]))
    assert z["loss"][0] == 0.0 and math.isinf(z["nll"][0])
    assert np.all(z["grad"][0:4] == 0.0)
    np.testing.assert_array_equal(a["grad"][4:], z["grad"][4:])
    assert a["loss"][1] == z["loss"][1] and math.isfinite(a["loss"][1])


def test_zero_length_utterances(oracle_mod):
    rng = np.random.default_rng(4)
    lp = _lp(rng, 8, 4)
    lengths = [5, 0, 3]
    targets = np.array([[1, 2], [1, 0], [2, 0]])
    for zi in (False, True):
        r = oracle_mod.ctc_packed(lp, [0, 5, 5, 8], lengths, targets, [2, 1, 1], blank=3, zero_infinity=zi)
        assert r["loss"][1] == (0.0 if zi else math.inf)
        r0 = oracle_mod.ctc_packed(lp, [0, 5, 5, 8], lengths, targets, [2, 0, 1], blank=3, zero_infinity=zi)
        assert r0["loss"][1] == 0.0 and not math.copysign(1.0, r0["loss"][1]) < 0


def test_permutation_invariance(oracle_mod):
    b = W.tiny()
    r = oracle_mod.ctc_batch(b)
    perm = [2, 0, 3, 1]
    lp = b.log_probs.numpy()
    cu = b.cu_seqlens.numpy()
    rows = np.concatenate([np.arange(cu[p], cu[p] + int(b.lengths[p])) for p in perm])
    lens = b.lengths.numpy()[perm]
    cu2 = np.concatenate([[0], np.cumsum(lens)])
    r2 = oracle_mod.ctc_packed(lp[rows], cu2, lens, b.targets.numpy()[perm], b.target_lengths.numpy()[perm],
                               blank=b.blank)
    np.testing.assert_allclose(r2["loss"], r["loss"][perm], rtol=1e-13)
    np.testing.assert_allclose(r2["grad"], r["grad"][rows], atol=1e-14)


def test_padding_fillers_and_gaps(oracle_mod):
    # tight batch vs the same utterances with gap rows between them, a 32-wide junk-filled targets
    # buffer and two zero-length fillers at the end (the static-shape regime of a captured step)
    tight = W.make_batch([9, 7, 4], [[1, 2, 3, 1], [2, 2, 4], [4, 1]], 6, seed=17, blank=5)
    gapped = W.make_batch([9, 7, 4, 0, 0], [[1, 2, 3, 1], [2, 2, 4], [4, 1], [], []], 6, seed=17, blank=5,
                          width=32, gaps=[2, 3, 0, 1, 0], T_total=30)
    # same log probabilities on the owned rows
    cu = gapped.cu_seqlens
    lp_g = gapped.log_probs.clone()
    for b in range(3):
        r0, rt = int(cu[b]), int(tight.cu_seqlens[b])
        lp_g[r0:r0 + int(tight.lengths[b])] = tight.log_probs[rt:rt + int(tight.lengths[b])]
    gapped.log_probs = lp_g
    a = oracle_mod.ctc_batch(tight)
    g = oracle_mod.ctc_batch(gapped)
    np.testing.assert_allclose(g["loss"][:3], a["loss"], rtol=1e-13)
    assert np.all(g["loss"][3:] == 0.0)
    owned = np.zeros(30, dtype=bool)
    for b in range(3):
        r0, rt, n = int(cu[b]), int(tight.cu_seqlens[b]), int(tight.lengths[b])
        owned[r0:r0 + n] = True
        np.testing.assert_allclose(g["grad"][r0:r0 + n], a["grad"][rt:rt + n], atol=1e-14)
    assert np.all(g["grad"][~owned] == 0.0)


def test_reductions_and_weights(oracle_mod):
    b = W.tiny()
    none = oracle_mod.ctc_batch(b, reduction="none")
    s = oracle_mod.ctc_batch(b, reduction="sum")
    m = oracle_mod.ctc_batch(b, reduction="mean")
    U = b.target_lengths.numpy().astype(np.float64)
    np.testing.assert_allclose(s["reduced"], none["loss"].sum(), rtol=1e-14)
    np.testing.assert_allclose(m["reduced"], np.mean(none["loss"] / np.maximum(U, 1)), rtol=1e-14)
    np.testing.assert_allclose(s["grad"], none["grad"], atol=0)
    cu = b.cu_seqlens.numpy()
    for i in range(b.B):
        rows = slice(cu[i], cu[i] + int(b.lengths[i]))
        np.testing.assert_allclose(m["grad"][rows], none["grad"][rows] / (b.B * max(U[i], 1)), atol=1e-15)
    gs = np.array([0.5, -2.0, 0.0, 3.0])
    w = oracle_mod.ctc_batch(b, reduction="none", grad_scale=gs)
    for i in range(b.B):
        rows = slice(cu[i], cu[i] + int(b.lengths[i]))
        np.testing.assert_allclose(w["grad"][rows], none["grad"][rows] * gs[i], atol=1e-14)


def test_zero_infinity_mean_counts_zeroed_utterances(oracle_mod):
    b = W.make_batch([3, 10], [[1, 1, 1], [1, 2]], 4, seed=2, zero_infinity=True, reduction="mean")
    r = oracle_mod.ctc_batch(b)
    assert r["loss"][0] == 0.0
    np.testing.assert_allclose(r["reduced"], (0.0 + r["loss"][1] / 2) / 2, rtol=1e-14)


@pytest.mark.parametrize("name", ["tiny", "small", "char_level"])
def test_workloads_run(oracle_mod, name):
    b = W.make_workload(name)
    r = oracle_mod.ctc_batch(b, want_grad=name != "char_level")
    assert np.all(np.isfinite(r["loss"]))


def test_asr_bpe_infeasible_selection(oracle_mod):
    b = W.asr_bpe()
    r = oracle_mod.ctc_batch(b, want_grad=False)
    bad = set(b.meta["infeasible"])
    assert len(bad) == 3
    for i in range(b.B):
        assert math.isinf(r["nll"][i]) == (i in bad)
        if i in bad:
            assert r["loss"][i] == 0.0


# --- planted mistakes: each mutation of the oracle source must be caught by the brute-force pin ---

_MUTATIONS = {
    "skip_allowed_for_repeats": ("l != ext_label(tgt, s - 2, blank)", "1"),
    "no_skip": ("skip = prev[s - 2];", "skip = -INFINITY;"),
    "advance_dropped": ("double advance = s >= 1 ? prev[s - 1] : -INFINITY;", "double advance = -INFINITY;"),
    "start_only_blank": ("if (S > 1) alpha[1] = lp[ext_label(tgt, 1, blank)];", ""),
    "end_only_last": ("double nll = -logsumexp3(last[S - 1], S >= 2 ? last[S - 2] : -INFINITY, -INFINITY);",
                      "double nll = -logsumexp3(last[S - 1], -INFINITY, -INFINITY);"),
    "beta_skip_wrong_side": ("l != ext_label(tgt, s + 2, blank)) skip = next[s + 2];",
                             "l != ext_label(tgt, s + 2, blank)) skip = next[s + 1];"),
    "posterior_sign": ("g[l] -= w * post;", "g[l] += w * post;"),
    "emission_not_removed": ("exp(alpha[t * S + s] + beta[t * S + s] - row[l] + n)",
                             "exp(alpha[t * S + s] + beta[t * S + s] + n)"),
    "emission_wrong_frame": ("cur[s] = logsumexp3(stay, advance, skip) + row[l];\n        }\n    }\n    /* step 4",
                             "cur[s] = logsumexp3(stay, advance, skip) + (row - D)[l];\n        }\n    }\n    /* step 4"),
}


@pytest.mark.parametrize("name", sorted(_MUTATIONS))
def test_pins_catch_planted_mistake(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ctc_oracle.c")).read()
    old, new = _MUTATIONS[name]
    assert old in src, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(mutated), "-o", str(so), "-lm"])
    lib = oracle.load_library(str(so))
    rng = np.random.default_rng(2024)
    caught = False
    for _ in range(40):
        T = int(rng.integers(1, 7))
        D = int(rng.integers(2, 4))
        U = int(rng.integers(0, 4))
        tgt = [int(x) for x in rng.integers(1, D, size=U)]
        lp = _lp(rng, T, D, 1.5)
        nll, post = brute.ctc_brute_states(lp, tgt, 0)
        tg = np.array([tgt], dtype=np.int64) if U else np.zeros((1, 0), np.int64)
        r = oracle.ctc_packed(lp, [0, T], [T], tg, [U], blank=0, lib=lib)
        if math.isinf(nll):
            caught |= not math.isinf(r["nll"][0])
            continue
        ok = np.isfinite(r["nll"][0]) and abs(r["nll"][0] - nll) < 1e-9 and np.allclose(
            r["grad"], np.exp(lp) - post, atol=1e-9)
        caught |= not ok
        if caught:
            break
    assert caught, f"planted mistake {name} was not detected"


def _mean_clamp_case():
    # utterance 0 has no labels (U = 0: the mean divides its loss by max(U, 1) = 1), utterance 1 has
    # two, utterance 2 one; values from the closed form of the empty target and from torch's CTC loss
    return W.make_batch([6, 9, 4], [[], [1, 2], [3]], 5, seed=21, sigma=1.3, reduction="mean")


def _check_mean_clamp(r, b):
    """The loss module's mean (PR page, `ctc.py` `forward_packed`): each loss over its target length
    clamped to at least 1, then the batch mean; the gradient weight of utterance b is 1 / (B max(U_b, 1)).
    Expected values come from the U = 0 closed form (loss = -sum_t lp[t][blank], posterior all on the
    blank) and from torch's float64 CTC loss, not from the oracle itself."""
    import torch.nn.functional as F

    lp = b.log_probs.double()
    cu = b.cu_seqlens.numpy()
    B = b.B
    U = [int(u) for u in b.target_lengths]
    losses = []
    for i in range(B):
        T = int(b.lengths[i])
        rows = lp[cu[i]:cu[i] + T]
        if U[i] == 0:
            losses.append(float(-rows[:, b.blank].sum()))
        else:
            losses.append(float(F.ctc_loss(rows[:, None, :], b.targets[i:i + 1, :U[i]], [T], [U[i]], blank=b.blank,
                                           reduction="none")[0]))
    want = sum(l / max(u, 1) for l, u in zip(losses, U)) / B
    np.testing.assert_allclose(r["reduced"], want, rtol=1e-12)
    T0 = int(b.lengths[0])
    rows0 = lp[cu[0]:cu[0] + T0].numpy()
    onehot = np.zeros_like(rows0)
    onehot[:, b.blank] = 1.0
    np.testing.assert_allclose(r["grad"][cu[0]:cu[0] + T0], (np.exp(rows0) - onehot) / (B * 1), atol=1e-14)


def test_mean_clamps_empty_target_length(oracle_mod):
    b = _mean_clamp_case()
    _check_mean_clamp(oracle_mod.ctc_batch(b), b)


@pytest.mark.parametrize("site", ["weight", "reduced"])
def test_mean_clamp_pin_catches_unclamped_divisor(tmp_path, site):
    # planted mistake: the mean divides by U instead of max(U, 1) (in the gradient weight, or in the
    # reduced loss); the pin above must reject the mutated oracle
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ctc_oracle.c")).read()
    old = {"weight": "w /= (double)B * (double)(U > 1 ? U : 1);",
           "reduced": "total += l / (double)(U > 1 ? U : 1);"}[site]
    assert old in src
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, old.replace("(U > 1 ? U : 1)", "U"), 1))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(mutated), "-o", str(so), "-lm"])
    lib = oracle.load_library(str(so))
    b = _mean_clamp_case()
    r = oracle.ctc_packed(b.log_probs, b.cu_seqlens, b.lengths, b.targets, b.target_lengths, blank=b.blank,
                          reduction="mean", lib=lib)
    with pytest.raises(AssertionError):
        _check_mean_clamp(r, b)


# --- NaN inputs (a reading: the pages do not treat them) ---------------------------------------------
# A NaN at the blank or a label column of an owned row makes the loss NaN and, under a non-zero weight,
# every column of the utterance's rows NaN (zero_infinity leaves a NaN loss alone); a NaN at another
# column shows only in that gradient entry; a zero weight gives zero rows.  Where the NaN lies on a
# state that some alignment passes through, or outside the label columns, torch's float64 CTC loss and
# gradient give the same and pin the oracle.  Where no alignment exists, torch's answer depends on the
# frame of the NaN (NaN or +inf, from the window of states it evaluates); there the reading alone fixes
# the expected values: loss NaN, rows NaN.

def _nan_cases():
    rng = np.random.default_rng(77)
    tg = [1, 1, 2]  # U = 3 with one repeat: at least 4 frames
    cases = []
    for label, T, at, zero_inf in [("label column on an alignment", 6, (2, 1), False),
                                   ("blank column on an alignment", 6, (1, 0), False),
                                   ("other column", 6, (3, 4), False),
                                   ("label column on an alignment, zero_infinity", 6, (4, 2), True),
                                   ("label column, no alignment", 3, (1, 1), False),
                                   ("label column, no alignment, zero_infinity", 3, (0, 1), True)]:
        lp = _lp(rng, T, 5, 1.2)
        lp[at] = np.nan
        cases.append((label, lp, tg, zero_inf))
    return cases


def _check_nan_case(lib, label, lp, tg, zero_inf):
    import torch.nn.functional as F

    T = lp.shape[0]
    r = oracle.ctc_packed(lp, [0, T], [T], np.array([tg], np.int64), [len(tg)], blank=0, zero_infinity=zero_inf,
                          lib=lib)
    got_loss = float(r["loss"][0])
    if "no alignment" in label:
        assert math.isnan(got_loss) and np.all(np.isnan(r["grad"])), label
        return
    x = torch.tensor(lp, dtype=torch.float64)[:, None, :].requires_grad_(True)
    loss = F.ctc_loss(x, torch.tensor([tg]), [T], [len(tg)], blank=0, reduction="none", zero_infinity=zero_inf)
    loss.sum().backward()
    want_loss = float(loss.detach()[0])
    want_grad = x.grad[:, 0].numpy()
    assert math.isnan(got_loss) == math.isnan(want_loss), label
    if not math.isnan(want_loss):
        np.testing.assert_allclose(got_loss, want_loss, rtol=1e-12, err_msg=label)
    assert np.array_equal(np.isnan(r["grad"]), np.isnan(want_grad)), label
    ok = ~np.isnan(want_grad)
    np.testing.assert_allclose(r["grad"][ok], want_grad[ok], atol=1e-12, err_msg=label)


def test_nan_inputs(oracle_mod):
    for case in _nan_cases():
        _check_nan_case(None, *case)


def test_zero_weight_gives_zero_rows_whatever_the_inputs(oracle_mod):
    rng = np.random.default_rng(78)
    lp = _lp(rng, 6, 5, 1.2)
    lp[2, 4] = np.nan   # a column no state reads
    lp[3, 1] = np.inf   # and one that exp() turns into inf
    r = oracle.ctc_packed(lp, [0, 6], [6], np.array([[1, 2]], np.int64), [2], blank=0,
                          grad_scale=np.zeros(1))
    assert np.all(r["grad"] == 0.0)


def test_nan_pin_catches_a_dropped_nan_rule(tmp_path):
    # planted mistake: the NaN scan no longer marks the loss; the pins above must reject the oracle
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ctc_oracle.c")).read()
    old = "{ n = NAN; break; }"
    assert old in src
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, "{ break; }", 1))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(mutated), "-o", str(so), "-lm"])
    lib = oracle.load_library(str(so))
    failures = 0
    for case in _nan_cases():
        try:
            _check_nan_case(lib, *case)
        except AssertionError:
            failures += 1
    assert failures > 0
