"""Seeded synthetic inputs for packed CTC: the five workload shapes and small structured cases.

This module only draws inputs (frame counts, target lengths, label ids, logits) and turns logits
into log probabilities with a float64 log-softmax rounded once to the storage dtype.  It holds none
of the CTC arithmetic, so both the HIP path and the float64 oracle can take their inputs from it.

Draw order for every workload, from ``numpy.random.default_rng(seed)``:
frame counts T_i (all utterances) -> target lengths U_i (all) -> label ids (utterance by
utterance, left to right) -> the infeasible selection (ASR-shaped case only) -> logits (float32,
row-major over ``(T_total, D)``, drawn in row chunks).

Readings of the workload descriptions (they only shape sizes and values):
``N(0, sigma)`` draws with standard deviation ``sigma``; an integer "uniform in [a, b]" is
inclusive, with fractional bounds rounded inward; ``round`` is round-half-to-even; "x% chance of
repeating the previous label" copies the previous id with probability x and otherwise draws fresh.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["PackedBatch", "WORKLOADS", "make_workload", "make_batch", "log_softmax_rounded"]

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64}


@dataclass
class PackedBatch:
    """A packed CTC batch on the CPU.

    ``log_probs`` is ``(T_total, D)`` in the storage dtype; ``cu_seqlens`` is ``(B+1,)`` int32;
    ``lengths``, ``targets`` (``(B, W)``) and ``target_lengths`` are int64.  Utterance ``b`` owns
    rows ``[cu_seqlens[b], cu_seqlens[b] + lengths[b])``.
    """

    name: str
    log_probs: torch.Tensor
    cu_seqlens: torch.Tensor
    lengths: torch.Tensor
    targets: torch.Tensor
    target_lengths: torch.Tensor
    blank: int
    zero_infinity: bool
    reduction: str
    meta: dict = field(default_factory=dict)

    @property
    def T_total(self) -> int:
        return int(self.log_probs.shape[0])

    @property
    def D(self) -> int:
        return int(self.log_probs.shape[1])

    @property
    def B(self) -> int:
        return int(self.lengths.numel())


def log_softmax_rounded(logits: np.ndarray, dtype: str, chunk_rows: int = 4096) -> torch.Tensor:
    """float64 log-softmax over the last axis, rounded once (nearest-even) to ``dtype``."""
    out = torch.empty(logits.shape, dtype=_DTYPES[dtype])
    for r0 in range(0, logits.shape[0], chunk_rows):
        x = logits[r0:r0 + chunk_rows].astype(np.float64)
        peak = x.max(axis=1, keepdims=True)
        z = x - peak
        z -= np.log(np.exp(z).sum(axis=1, keepdims=True))
        out[r0:r0 + chunk_rows] = torch.from_numpy(z).to(_DTYPES[dtype])
    return out


def _draw_logits(rng: np.random.Generator, T_total: int, D: int, sigma: float, chunk_rows: int = 4096) -> np.ndarray:
    logits = np.empty((T_total, D), dtype=np.float32)
    for r0 in range(0, T_total, chunk_rows):
        n = min(chunk_rows, T_total - r0)
        logits[r0:r0 + n] = rng.normal(0.0, sigma, size=(n, D)).astype(np.float32)
    return logits


def _labels_with_repeats(rng, U, lo, hi, p_repeat):
    out = []
    for j in range(U):
        if j > 0 and p_repeat > 0 and rng.random() < p_repeat:
            out.append(out[-1])
        else:
            out.append(int(rng.integers(lo, hi + 1)))
    return out


def _zipf_sampler(n: int, a: float):
    """Inverse-CDF sampler for P(k) proportional to k**-a on 1..n."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-a)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]

    def draw(rng, size=None):
        u = rng.random(size)
        return np.searchsorted(cdf, u, side="right") + 1

    return draw


def _pack(name, rng, Ts, labels, D, sigma, dtype, blank, zero_infinity, reduction, meta=None):
    B = len(Ts)
    W = max([len(l) for l in labels] + [0])
    targets = torch.zeros((B, W), dtype=torch.int64)
    for b, l in enumerate(labels):
        if l:
            targets[b, : len(l)] = torch.tensor(l, dtype=torch.int64)
    lengths = torch.tensor(Ts, dtype=torch.int64)
    target_lengths = torch.tensor([len(l) for l in labels], dtype=torch.int64)
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lengths, 0).to(torch.int32)
    T_total = int(sum(Ts))
    logits = _draw_logits(rng, T_total, D, sigma)
    lp = log_softmax_rounded(logits, dtype)
    return PackedBatch(name, lp, cu, lengths, targets, target_lengths, blank, zero_infinity, reduction, meta or {})


def tiny(seed: int = 1) -> PackedBatch:
    """B=4, T_i in [20,50], D=16 (blank 0), U_i in [3,10], labels 1..15, N(0,1) logits, f32, none."""
    rng = np.random.default_rng(seed)
    B, D = 4, 16
    Ts = [int(t) for t in rng.integers(20, 51, size=B)]
    Us = [int(u) for u in rng.integers(3, 11, size=B)]
    labels = [[int(x) for x in rng.integers(1, 16, size=U)] for U in Us]
    return _pack("tiny", rng, Ts, labels, D, 1.0, "f32", 0, False, "none")


def small(seed: int = 2) -> PackedBatch:
    """B=32, T_i in [200,800], D=128, U_i in [T/8, T/4], labels 1..127 with 10% repeats, N(0,2), f32, mean."""
    rng = np.random.default_rng(seed)
    B, D = 32, 128
    Ts = [int(t) for t in rng.integers(200, 801, size=B)]
    Us = [int(rng.integers(math.ceil(T / 8), T // 4 + 1)) for T in Ts]
    labels = [_labels_with_repeats(rng, U, 1, 127, 0.10) for U in Us]
    return _pack("small", rng, Ts, labels, D, 2.0, "f32", 0, False, "mean")


def asr_bpe(seed: int = 3) -> PackedBatch:
    """B=64, T_i in [100,1500], D=1025, U_i=round(T/4*U(0.7,1)), Zipf(1.1) labels, N(0,3), bf16,
    5% infeasible targets, zero_infinity, sum.

    Infeasible reading: exactly round(0.05*B) utterances (chosen by a permutation) get
    ``U = floor((T+3)/2)`` copies of one Zipf-drawn id, so U + (U-1) repeats exceeds T while U <= T.
    """
    rng = np.random.default_rng(seed)
    B, D = 64, 1025
    Ts = [int(t) for t in rng.integers(100, 1501, size=B)]
    Us = [int(np.rint(T / 4 * rng.uniform(0.7, 1.0))) for T in Ts]
    zipf = _zipf_sampler(1024, 1.1)
    labels = [[int(x) for x in zipf(rng, U)] for U in Us]
    n_bad = int(np.rint(0.05 * B))
    bad = [int(i) for i in rng.permutation(B)[:n_bad]]
    for i in bad:
        U = (Ts[i] + 3) // 2
        labels[i] = [int(zipf(rng))] * U
    return _pack("asr_bpe", rng, Ts, labels, D, 3.0, "bf16", 0, True, "sum", {"infeasible": sorted(bad)})


def large_vocab(seed: int = 4) -> PackedBatch:
    """B=16, T_i in [500,3000], D=8193, U_i=round(T/6), labels 1..8192, N(0,3), f16, mean."""
    rng = np.random.default_rng(seed)
    B, D = 16, 8193
    Ts = [int(t) for t in rng.integers(500, 3001, size=B)]
    Us = [int(np.rint(T / 6)) for T in Ts]
    labels = [[int(x) for x in rng.integers(1, 8193, size=U)] for U in Us]
    return _pack("large_vocab", rng, Ts, labels, D, 3.0, "f16", 0, False, "mean")


def char_level(seed: int = 5) -> PackedBatch:
    """B=128, T_i=clip(round(lognormal(5.2,0.6)),50,1200), D=29, U_i in [0.35T,0.48T], labels 1..28 with
    25% repeats, N(0,2), f32, mean, zero_infinity."""
    rng = np.random.default_rng(seed)
    B, D = 128, 29
    Ts = [int(t) for t in np.clip(np.rint(rng.lognormal(5.2, 0.6, size=B)), 50, 1200)]
    Us = [int(rng.integers(math.ceil(0.35 * T), math.floor(0.48 * T) + 1)) for T in Ts]
    labels = [_labels_with_repeats(rng, U, 1, 28, 0.25) for U in Us]
    return _pack("char_level", rng, Ts, labels, D, 2.0, "f32", 0, True, "mean")


WORKLOADS = {
    "tiny": tiny,
    "small": small,
    "asr_bpe": asr_bpe,
    "large_vocab": large_vocab,
    "char_level": char_level,
}


def make_workload(name: str, seed: int | None = None) -> PackedBatch:
    fn = WORKLOADS[name]
    return fn() if seed is None else fn(seed)


def make_batch(
    lengths,
    target_lists,
    D: int,
    *,
    seed: int = 0,
    sigma: float = 1.0,
    dtype: str = "f32",
    blank: int = 0,
    zero_infinity: bool = False,
    reduction: str = "none",
    width: int | None = None,
    gaps=None,
    junk_fill: int | None = None,
    T_total: int | None = None,
    name: str = "custom",
) -> PackedBatch:
    """A structured batch: explicit frame counts and targets, random logits.

    ``gaps`` (optional, one per utterance) inserts that many unowned rows before each utterance;
    ``width`` over-allocates the targets buffer, filled past each length with ``junk_fill``
    (or random ids when ``junk_fill`` is None); ``T_total`` may add unowned rows at the end.
    """
    rng = np.random.default_rng(seed)
    B = len(lengths)
    gaps = list(gaps) if gaps is not None else [0] * B
    starts, pos = [], 0
    for b in range(B):
        pos += int(gaps[b])
        starts.append(pos)
        pos += int(lengths[b])
    total = pos if T_total is None else int(T_total)
    assert total >= pos
    W = max([len(t) for t in target_lists] + [0]) if width is None else int(width)
    targets = torch.zeros((B, W), dtype=torch.int64)
    if W:
        fill = rng.integers(0, D, size=(B, W)) if junk_fill is None else np.full((B, W), junk_fill)
        targets[:] = torch.from_numpy(np.asarray(fill, dtype=np.int64))
    for b, t in enumerate(target_lists):
        if len(t):
            targets[b, : len(t)] = torch.tensor(list(t), dtype=torch.int64)
    cu = torch.zeros(B + 1, dtype=torch.int32)
    # cu_seqlens[b] is the first row of utterance b; the final entry closes the buffer
    if B:
        cu[:B] = torch.tensor(starts, dtype=torch.int32)
    cu[B] = total
    logits = _draw_logits(rng, total, D, sigma)
    lp = log_softmax_rounded(logits, dtype)
    return PackedBatch(
        name,
        lp,
        cu,
        torch.tensor([int(x) for x in lengths], dtype=torch.int64),
        targets,
        torch.tensor([len(t) for t in target_lists], dtype=torch.int64),
        blank,
        zero_infinity,
        reduction,
    )
