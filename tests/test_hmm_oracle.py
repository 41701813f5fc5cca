"""Pins of the float64 HMM oracle (the POPCORNBENCH page's log-space forward of an HMM module with
normalised initial, transition and emission log weights) against things other than itself:
enumeration of every state path on tiny cases (asymmetric transitions, so a transposed matrix or a
wrong normalisation axis fails), and closed forms (uniform parameters; a single state)."""

import numpy as np
import pytest

from oracle import hmm


@pytest.mark.parametrize("S,O,T,B,seed", [(1, 3, 4, 2, 0), (2, 2, 1, 3, 1), (3, 4, 4, 4, 2), (4, 3, 3, 3, 3),
                                          (3, 5, 5, 2, 4)])
def test_brute_force_paths(S, O, T, B, seed):
    rng = np.random.default_rng(seed)
    li, lt, le = rng.normal(0, 2, size=S), rng.normal(0, 2, size=(S, S)), rng.normal(0, 2, size=(S, O))
    lt[0, -1] += 3.0  # asymmetric on purpose
    obs = rng.integers(0, O, size=(B, T))
    np.testing.assert_allclose(hmm.hmm_model_loglik(li, lt, le, obs), hmm.hmm_model_loglik_brute(li, lt, le, obs),
                               rtol=1e-12, atol=1e-12)


def test_uniform_parameters_closed_form():
    # every state equally likely and every symbol equally likely from every state: log(1/O) per frame
    S, O, T = 16, 64, 128
    rng = np.random.default_rng(5)
    obs = rng.integers(0, O, size=(6, T))
    got = hmm.hmm_model_loglik(np.full(S, 0.3), np.full((S, S), -1.7), np.full((S, O), 2.0), obs)
    np.testing.assert_allclose(got, T * np.log(1.0 / O), rtol=1e-13)


def test_single_state_closed_form():
    # one state: the likelihood is the product of its emission probabilities
    rng = np.random.default_rng(6)
    le = rng.normal(0, 1, size=(1, 7))
    obs = rng.integers(0, 7, size=(3, 9))
    logB = le[0] - np.log(np.exp(le[0]).sum())
    want = logB[obs].sum(axis=1)
    np.testing.assert_allclose(hmm.hmm_model_loglik(np.zeros(1), np.zeros((1, 1)), le, obs), want, rtol=1e-13)
