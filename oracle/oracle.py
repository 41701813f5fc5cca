"""ctypes front end of the float64 CPU oracle (``ctc_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg use it to
check and to time the HIP path.  It never feeds the HIP path and shares no code with it.
The oracle's steps and citations are in the header of ``ctc_oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ctc_oracle.c")
_LIB = os.path.join(_HERE, "libctc_oracle.so")

RED = {"none": 0, "sum": 1, "mean": 2}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math: IEEE float64 throughout)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load_library(path: str):
    """Load an oracle build from ``path`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.ctc_oracle.argtypes = [P, I64, I64, P, P, I64, P, I64, P, I64, ctypes.c_int, ctypes.c_int, P, P, P, P, P,
                               ctypes.c_int]
    lib.ctc_oracle.restype = ctypes.c_int
    lib.ctc_oracle_posteriors.argtypes = [P, I64, I64, P, I64, I64, P, P, P, P]
    lib.ctc_oracle_posteriors.restype = ctypes.c_double
    lib.ctc_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = load_library(build())
    return _lib


def max_threads() -> int:
    return int(_load().ctc_oracle_max_threads())


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return np.ascontiguousarray(x.detach().cpu().to(torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return np.ascontiguousarray(x.detach().cpu().to(torch.int64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def ctc_packed(log_probs, cu_seqlens, lengths, targets, target_lengths, *, blank: int, zero_infinity: bool = False,
               reduction: str = "none", grad_scale=None, want_grad: bool = True, nthreads: int = 0,
               lib=None) -> dict:
    """Loss, reduced loss and gradient of a packed batch in float64.

    bf16/f16/f32 log probabilities are upcast exactly.  Returns a dict with ``nll`` (raw, +inf when
    no alignment exists), ``loss`` (after zero_infinity), ``reduced`` (sum/mean, else None) and
    ``grad`` ((T_total, D) float64 with the reduction's weights, or None).  ``lib`` selects another
    build of the same source (the mutation tests use it).
    """
    lib = _load() if lib is None else lib
    lp = _f64(log_probs)
    if lp.ndim != 2:
        raise ValueError("log_probs must be (T_total, D)")
    T_total, D = lp.shape
    len_ = _i64(lengths)
    B = len_.shape[0]
    cu = _i64(cu_seqlens)[:B]
    cu = np.ascontiguousarray(cu)
    tg = _i64(targets)
    if tg.ndim != 2:
        tg = tg.reshape(B, -1)
    W = tg.shape[1]
    tl = _i64(target_lengths)
    gs = None if grad_scale is None else _f64(grad_scale)
    nll = np.empty(B, dtype=np.float64)
    loss = np.empty(B, dtype=np.float64)
    red = np.empty(1, dtype=np.float64)
    grad = np.empty((T_total, D), dtype=np.float64) if want_grad else None
    rc = lib.ctc_oracle(_ptr(lp), T_total, D, _ptr(cu), _ptr(len_), B, _ptr(tg), W, _ptr(tl), int(blank),
                        int(bool(zero_infinity)), RED[reduction], _ptr(gs), _ptr(nll), _ptr(loss), _ptr(red),
                        _ptr(grad), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return {"nll": nll, "loss": loss, "reduced": None if reduction == "none" else float(red[0]), "grad": grad}


def ctc_batch(batch, *, reduction: str | None = None, grad_scale=None, want_grad: bool = True, nthreads: int = 0):
    """``ctc_packed`` on a ``workloads.PackedBatch``."""
    return ctc_packed(batch.log_probs, batch.cu_seqlens, batch.lengths, batch.targets, batch.target_lengths,
                      blank=batch.blank, zero_infinity=batch.zero_infinity,
                      reduction=batch.reduction if reduction is None else reduction, grad_scale=grad_scale,
                      want_grad=want_grad, nthreads=nthreads)


def posteriors(log_probs_utt, targets_utt, blank: int) -> dict:
    """State posteriors of ONE utterance: ``gamma`` = exp(alpha + beta - lp + nll) and ``gamma_norm``
    (the per-frame softmax over states of alpha + beta - lp), both (T, S); also alpha, beta, nll."""
    lib = _load()
    lp = _f64(log_probs_utt)
    T, D = lp.shape
    tg = _i64(targets_utt).reshape(-1)
    U = tg.shape[0]
    S = 2 * U + 1
    g = np.zeros((max(T, 1), S))
    gn = np.zeros((max(T, 1), S))
    a = np.zeros((max(T, 1), S))
    b = np.zeros((max(T, 1), S))
    nll = lib.ctc_oracle_posteriors(_ptr(lp), D, T, _ptr(tg if U else np.zeros(1, np.int64)), U, int(blank), _ptr(g),
                                    _ptr(gn), _ptr(a), _ptr(b))
    return {"gamma": g[:T], "gamma_norm": gn[:T], "alpha": a[:T], "beta": b[:T], "nll": float(nll)}
