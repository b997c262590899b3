"""Pins for the oracle's hybrid (window + linear state + sparse cache) prefill.

The pages fix the three memories and the refresh steps (LoLA page,
Metodologia and Estratégia de Inferência) but not the block timing, the
normalisation or tie order; those are readings. They are pinned here by
special cases that reduce to textbook routines (plain causal softmax;
window + exact squared-kernel attention when the cache is empty) and by a
second, token-by-token enumeration of the refresh chain whose scores come
from the brute-force self-recall error.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle as O


def _data(T, d, seed, dup=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    for t in rng.choice(np.arange(1, T), dup, replace=False) if dup else []:
        k[t] = k[rng.integers(0, t)] + 0.05 * rng.standard_normal(d)
    v = rng.standard_normal((T, d))
    return q, k, v


def _causal_softmax(q, k, v, scale):
    T = len(q)
    out = np.zeros_like(v)
    for t in range(T):
        p = softmax(scale * (k[: t + 1] @ q[t]))
        out[t] = p @ v[: t + 1]
    return out


@pytest.mark.parametrize("W,lam", [(16, 1000), (1000, 4), (1000, 1000)])
def test_no_fold_reduces_to_causal_softmax(W, lam):
    q, k, v = _data(150, 6, 1)
    scale = 1 / math.sqrt(6)
    r = O.hybrid_prefill(q, k, v, window=W, cache_size=lam, refresh=8, scale=scale)
    np.testing.assert_allclose(r["o"], _causal_softmax(q, k, v, scale), rtol=1e-12, atol=1e-13)
    assert r["refreshes"] == 0 and np.all(r["H"] == 0)


@pytest.mark.parametrize("W,R", [(16, 8), (24, 8), (32, 16)])
def test_empty_cache_is_window_plus_squared_kernel(W, R):
    # cache_size = 0: every evicted token is folded at once, so
    # o_t = [sum_{i in [f,t]} e^{s q.k_i} v_i + sum_{i<f} (q.k_i)^2 v_i] / [same without v]
    q, k, v = _data(140, 5, 2)
    scale = 0.7
    r = O.hybrid_prefill(q, k, v, window=W, cache_size=0, refresh=R, scale=scale)
    T = len(q)
    want = np.zeros_like(v)
    for t in range(T):
        f = max(0, (t // R) * R - W)
        w1 = np.exp(scale * (k[f: t + 1] @ q[t]))
        w2 = (k[:f] @ q[t]) ** 2
        want[t] = (w1 @ v[f: t + 1] + w2 @ v[:f]) / (w1.sum() + w2.sum())
    np.testing.assert_allclose(r["o"], want, rtol=1e-11, atol=1e-12)


def _hybrid_token_by_token(q, k, v, W, lam, R, scale):
    """Second enumeration: per-token membership, scores from pairs."""
    T = len(q)
    member = np.zeros(T, dtype=int)  # 0 = not yet seen / window, 1 = cache, 2 = folded
    f_prev = 0
    trace = {}
    o = np.zeros_like(v)
    f = 0
    for t in range(T):
        if t % R == 0:
            f = max(0, t - W)
            newly = list(range(f_prev, f))
            f_prev = f
            for i in newly:
                member[i] = 1
            cached = [i for i in range(T) if member[i] == 1]
            if newly and len(cached) > lam:
                folded = [i for i in range(T) if member[i] == 2]
                sc = O.sre_bruteforce(k[folded], v[folded], k[cached], v[cached])
                order = sorted(range(len(cached)), key=lambda j: (-sc[j], cached[j]))
                keep = sorted(cached[j] for j in order[:lam])
                for i in cached:
                    if i not in keep:
                        member[i] = 2
                trace[t // R] = keep
        num = np.zeros(v.shape[1])
        den = 0.0
        for i in range(t + 1):
            if i >= f or member[i] == 1:
                w = math.exp(scale * float(q[t] @ k[i]))
            else:
                w = float(q[t] @ k[i]) ** 2
            num += w * v[i]
            den += w
        o[t] = num / den
    cache = [i for i in range(T) if member[i] == 1]
    return o, trace, cache


# refresh = 1 is the token-by-token decode: one eviction and at most one fold per token
@pytest.mark.parametrize("seed,W,lam,R", [(3, 16, 4, 8), (4, 24, 6, 8), (5, 8, 3, 4), (6, 8, 3, 1),
                                         (7, 0, 2, 1), (8, 5, 0, 1)])
def test_refresh_chain_against_token_by_token_enumeration(seed, W, lam, R):
    q, k, v = _data(120, 4, seed, dup=10)
    scale = 0.5
    r = O.hybrid_prefill(q, k, v, window=W, cache_size=lam, refresh=R, scale=scale)
    o2, trace2, cache2 = _hybrid_token_by_token(q, k, v, W, lam, R, scale)
    assert r["trace"].keys() == trace2.keys() and len(trace2) > 3
    for b in trace2:
        assert r["trace"][b] == trace2[b]
    assert r["cache"] == cache2
    np.testing.assert_allclose(r["o"], o2, rtol=1e-10, atol=1e-12)


def test_first_refresh_scores_against_empty_state():
    # the first scored refresh sees an empty linear state: SRE = ||v||^2, so
    # the largest-norm values stay cached.
    q, k, v = _data(64, 3, 6)
    r = O.hybrid_prefill(q, k, v, window=8, cache_size=4, refresh=4, scale=1.0)
    first = min(r["trace"])
    cand = list(range(0, (first * 4) - 8))
    norms = np.sum(v[cand] ** 2, axis=1)
    want = sorted(np.array(cand)[O.select_topk(norms, 4, ids=np.array(cand))].tolist())
    assert r["trace"][first] == want
