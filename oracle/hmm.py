"""Generic dense log-space HMM forward, applied to the CTC topology.

TEST INFRASTRUCTURE ONLY.  An independent route to the CTC likelihood: the POPCORNBENCH page on a
log-space HMM forward kernel describes the forward algorithm with a dense S x S log-transition
matrix: alpha_0 = initial + emission of the first observation, then
alpha_t[j] = logsumexp_i(alpha_{t-1}[i] + A[i, j]) + emission_t[j], and the sequence log-likelihood is
the log-sum-exp of the last alpha over the accepting states.  CTC is the special case whose states
are the extended label sequence (blank, l1, blank, ..., lU, blank), whose transitions are stay,
advance by one, and skip by two into a label that differs from the label two states back, whose
initial mass sits on the first two states and whose accepting states are the last two.
Nothing here shares code with the banded recursion in ``ctc_oracle.c``.

``hmm_model_loglik`` is the page's HMM module itself (normalised initial, transition and emission
log weights, then the forward per observation sequence), the reference for the GPU HMM forward;
it is pinned by enumeration of every state path and by closed forms (tests/test_hmm_oracle.py).
"""

from __future__ import annotations

import numpy as np


def ctc_topology(target, blank: int):
    """Extended labels, dense log-transition matrix, log-initial and accepting mask for one target."""
    ext = [blank]
    for l in target:
        ext += [int(l), blank]
    S = len(ext)
    A = np.full((S, S), -np.inf)
    for i in range(S):
        A[i, i] = 0.0
        if i + 1 < S:
            A[i, i + 1] = 0.0
        j = i + 2
        if j < S and j % 2 == 1 and ext[j] != ext[i]:
            A[i, j] = 0.0
    init = np.full(S, -np.inf)
    init[0] = 0.0
    if S > 1:
        init[1] = 0.0
    accept = np.zeros(S, dtype=bool)
    accept[S - 1] = True
    if S > 1:
        accept[S - 2] = True
    return ext, A, init, accept


def _lse(x, axis=None):
    m = np.max(x, axis=axis, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = m_safe + np.log(np.sum(np.exp(x - m_safe), axis=axis, keepdims=True))
    out = np.where(np.isneginf(m), -np.inf, out)
    return np.squeeze(out, axis=axis) if axis is not None else out.reshape(())


def hmm_forward_loglik(log_emissions: np.ndarray, log_trans: np.ndarray, log_init: np.ndarray, accept) -> float:
    """Dense forward: log_emissions (T, S), log_trans (S, S) with A[i, j] = log P(j | i)."""
    T = log_emissions.shape[0]
    alpha = log_init + log_emissions[0]
    for t in range(1, T):
        alpha = _lse(alpha[:, None] + log_trans, axis=0) + log_emissions[t]
    return float(_lse(alpha[np.asarray(accept)]))


def ctc_nll_via_hmm(lp: np.ndarray, target, blank: int) -> float:
    lp = np.asarray(lp, dtype=np.float64)
    if lp.shape[0] == 0:
        return 0.0 if len(target) == 0 else np.inf
    ext, A, init, accept = ctc_topology(target, blank)
    emis = lp[:, ext]
    return -hmm_forward_loglik(emis, A, init, accept)


def _normalise(x: np.ndarray, axis: int) -> np.ndarray:
    return x - _lse(x, axis=axis)[..., None] if x.ndim > 1 else x - _lse(x)


def hmm_model_loglik(log_init, log_trans, log_emit, observations) -> np.ndarray:
    """The POPCORNBENCH page's HMM module, in float64: normalise the initial log weights over states,
    each transition row over next states and each emission row over symbols (subtract the
    log-sum-exp), then per sequence alpha_0 = log_pi + log_B[:, o_0],
    alpha_t[j] = logsumexp_i(alpha_{t-1}[i] + log_A[i, j]) + log_B[j, o_t], and the log-likelihood is
    the log-sum-exp of the last alpha over all states.  observations (B, T) ints; returns (B,)."""
    li = np.asarray(log_init, dtype=np.float64)
    lt = np.asarray(log_trans, dtype=np.float64)
    le = np.asarray(log_emit, dtype=np.float64)
    obs = np.asarray(observations, dtype=np.int64)
    log_pi = li - _lse(li)
    log_A = _normalise(lt, 1)
    log_B = _normalise(le, 1)
    out = np.empty(obs.shape[0])
    for b in range(obs.shape[0]):
        emis = log_B[:, obs[b]].T  # (T, S)
        out[b] = hmm_forward_loglik(emis, log_A, log_pi, np.ones(log_A.shape[0], dtype=bool))
    return out


def hmm_model_loglik_brute(log_init, log_trans, log_emit, observations) -> np.ndarray:
    """The same quantity by enumerating every state path (tiny S and T only): log of the sum over
    paths of pi[s_0] B[s_0, o_0] prod_t A[s_{t-1}, s_t] B[s_t, o_t], normalised parameters."""
    import itertools

    li = np.asarray(log_init, dtype=np.float64)
    lt = np.asarray(log_trans, dtype=np.float64)
    le = np.asarray(log_emit, dtype=np.float64)
    pi = np.exp(li) / np.exp(li).sum()
    A = np.exp(lt) / np.exp(lt).sum(axis=1, keepdims=True)
    Bm = np.exp(le) / np.exp(le).sum(axis=1, keepdims=True)
    obs = np.asarray(observations, dtype=np.int64)
    S, out = A.shape[0], []
    for seq in obs:
        tot = 0.0
        for path in itertools.product(range(S), repeat=len(seq)):
            p = pi[path[0]] * Bm[path[0], seq[0]]
            for t in range(1, len(seq)):
                p *= A[path[t - 1], path[t]] * Bm[path[t], seq[t]]
            tot += p
        out.append(np.log(tot))
    return np.array(out)
