"""Brute-force CTC by enumerating every frame-level path (tiny inputs only).

TEST INFRASTRUCTURE ONLY.  This is the definition of the CTC likelihood written out, with no
recursion: a path assigns one class to each of the T frames; it collapses to a label sequence by
merging runs of equal classes and then dropping the blank; the likelihood of a target is the sum,
over all paths that collapse to it, of the product of the per-frame probabilities.  The class
posterior of frame t is the share of that likelihood carried by the paths whose frame t holds the
class.  With log probabilities from a log-softmax, the gradient of the loss -log p with respect to
the logits is then exp(lp) - posterior per frame (the convention of the NeMo packed CTC kernel page,
whose gradient is the one with respect to the logits of a log-softmax).
"""

from __future__ import annotations

import itertools
import math

import numpy as np


def collapse(path, blank: int):
    out = []
    prev = None
    for c in path:
        if c != prev and c != blank:
            out.append(c)
        prev = c
    return out


def ctc_brute(lp: np.ndarray, target, blank: int):
    """lp: (T, D) float64 log probabilities of one utterance.  Returns (nll, class_posterior (T, D)).

    nll is +inf (and the posterior all zeros) when no path collapses to the target.
    """
    lp = np.asarray(lp, dtype=np.float64)
    T, D = lp.shape
    target = list(int(x) for x in target)
    if T == 0:
        return (0.0 if not target else math.inf), np.zeros((0, D))
    total = 0.0
    post = np.zeros((T, D))
    p = np.exp(lp)
    for path in itertools.product(range(D), repeat=T):
        if collapse(path, blank) != target:
            continue
        w = 1.0
        for t, c in enumerate(path):
            w *= p[t, c]
        total += w
        for t, c in enumerate(path):
            post[t, c] += w
    if total == 0.0:
        return math.inf, np.zeros((T, D))
    return -math.log(total), post / total


def count_alignments(T: int, U: int) -> int:
    """Number of length-T frame paths that collapse to a fixed U-label sequence without adjacent
    repeats: choose the 2U run boundaries among T+U positions (a stars-and-bars count)."""
    return math.comb(T + U, 2 * U)


def ctc_brute_states(lp: np.ndarray, target, blank: int):
    """Brute force over state paths of the extended label sequence (blank, l1, blank, ..., lU, blank).

    A state path starts in the first blank or the first label, moves at each frame by staying, by
    one state, or by two states into a label that differs from the label two states back (ids
    compared as ids, so a target equal to the blank id is an ordinary label state), and ends in the
    last label or the last blank.  Its weight is the product of the frame probabilities of the
    states' classes.  For targets without the blank id this is the same sum as ``ctc_brute``; with
    the blank id among the targets it is the quantity the packed kernel page's recursion computes.
    Returns (nll, class_posterior (T, D)).
    """
    lp = np.asarray(lp, dtype=np.float64)
    T, D = lp.shape
    ext = [blank]
    for l in target:
        ext += [int(l), blank]
    S = len(ext)
    if T == 0:
        return (0.0 if not target else math.inf), np.zeros((0, D))
    p = np.exp(lp)
    total = 0.0
    post = np.zeros((T, D))

    def moves(s):
        out = [s]
        if s + 1 < S:
            out.append(s + 1)
        if s + 2 < S and (s + 2) % 2 == 1 and ext[s + 2] != ext[s]:
            out.append(s + 2)
        return out

    stack = [([s], p[0, ext[s]]) for s in (0, 1) if s < S]
    while stack:
        path, w = stack.pop()
        if len(path) == T:
            if path[-1] >= S - 2:
                total += w
                for t, s in enumerate(path):
                    post[t, ext[s]] += w
            continue
        t = len(path)
        for n in moves(path[-1]):
            stack.append((path + [n], w * p[t, ext[n]]))
    if total == 0.0:
        return math.inf, np.zeros((T, D))
    return -math.log(total), post / total
