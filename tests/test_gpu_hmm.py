"""Dense log-space HMM forward on the GPU (hmm_forward_loglik through the C ABI) vs the float64
oracle of the POPCORNBENCH page's HMM module (oracle/hmm.py: hmm_model_loglik).

Tolerance: log-likelihoods within 1e-4 relative (the float32 bar of the loss), plus 1e-5 absolute.
Inputs are seeded and synthetic: normal(0, sigma) raw log weights (normalised inside the library,
as the module does) and uniform symbols; the page's size is S = 16, T = 128, B = 64, O = 64.
"""

import numpy as np
import pytest
import torch

from oracle import hmm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ctc_forward_backward_amd import api as _api

    _api._load()
    return _api


def _case(S, O, T, B, seed, sigma=1.0, i64=False, left_to_right=False):
    rng = np.random.default_rng(seed)
    li = rng.normal(0, sigma, size=S).astype(np.float32)
    lt = rng.normal(0, sigma, size=(S, S)).astype(np.float32)
    le = rng.normal(0, sigma, size=(S, O)).astype(np.float32)
    if left_to_right:  # structural zeros: only stay and advance
        mask = np.triu(np.ones((S, S), dtype=bool)) & ~np.triu(np.ones((S, S), dtype=bool), k=2)
        lt = np.where(mask, lt, -np.inf).astype(np.float32)
    obs = rng.integers(0, O, size=(B, T)).astype(np.int64 if i64 else np.int32)
    return li, lt, le, obs


def _run(api, li, lt, le, obs):
    dev = torch.device("cuda:0")
    out = api.hmm_forward(torch.from_numpy(li).to(dev), torch.from_numpy(lt).to(dev), torch.from_numpy(le).to(dev),
                          torch.from_numpy(obs).to(dev))
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


@pytest.mark.parametrize("S,O,T,B,seed,kw", [
    (16, 64, 128, 64, 1, {}),              # the page's size
    (16, 64, 128, 64, 2, {"sigma": 3.0}),
    (1, 5, 40, 3, 3, {}),
    (7, 9, 65, 5, 4, {}),                  # ragged state count, one symbol block boundary
    (33, 20, 200, 6, 5, {"i64": True}),    # the 64-state tile, three symbol blocks
    (64, 256, 130, 9, 6, {}),              # the widest state count and table
    (16, 1, 17, 4, 7, {}),                 # one symbol
    (12, 30, 1, 8, 8, {}),                 # one frame
    (10, 16, 90, 7, 9, {"left_to_right": True}),
])
def test_hmm_forward_vs_oracle(api, S, O, T, B, seed, kw):
    print(f"[gpu hmm] S={S} O={O} T={T} B={B} {kw}", flush=True)
    li, lt, le, obs = _case(S, O, T, B, seed, **kw)
    got = _run(api, li, lt, le, obs)
    ref = hmm.hmm_model_loglik(li, lt, le, obs)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-4, atol=1e-5)


def test_hmm_empty_batch(api):
    li, lt, le, obs = _case(4, 3, 5, 0, 10)
    assert _run(api, li, lt, le, obs).shape == (0,)
