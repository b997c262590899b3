"""Pins for the oracle's prefill gradients (CPU only).

The gradients are pinned by central finite differences of the forward
(brute-force form) and by identities that hold whatever the formula: the
output is invariant to scaling one query, invariant to scaling every key,
and linear in the values, so the matching directional derivatives are 0, 0
and the loss itself. The row-sampled form is pinned against the full one.
"""
import numpy as np
import pytest

import oracle as O


def _data(T, d, dv, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, dv)),
            rng.standard_normal((T, dv)))


def _loss(q, k, v, do, eps):
    return float(np.sum(do * O.prefill_bruteforce(q, k, v, eps=eps)))


@pytest.mark.parametrize("T,d,dv,eps", [(7, 3, 2, 0.0), (9, 4, 3, 0.3), (5, 2, 5, 0.0)])
def test_gradients_match_finite_differences(T, d, dv, eps):
    q, k, v, do = _data(T, d, dv, seed=T * 10 + d)
    dq, dk, dv_ = O.prefill_backward(q, k, v, do, eps=eps)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv_)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, eps)
            x[idx] = old - h
            lm = _loss(q, k, v, do, eps)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_homogeneity_identities():
    # eps = 0: o_t(a q_t) = o_t(q_t); o(a K) = o(K); o is linear in V
    T, d, dv = 40, 8, 6
    q, k, v, do = _data(T, d, dv, seed=5)
    dq, dk, dv_ = O.prefill_backward(q, k, v, do)
    np.testing.assert_allclose(np.sum(q * dq, axis=1), 0.0, atol=1e-10)
    np.testing.assert_allclose(np.sum(k * dk), 0.0, atol=1e-9)
    loss = float(np.sum(do * O.prefill_bruteforce(q, k, v)))
    np.testing.assert_allclose(np.sum(v * dv_), loss, rtol=1e-12)


def test_first_token_value_gradient_and_zero_rows():
    # o_0 = v_0 exactly, so a loss on token 0 alone gives dv_0 = do_0 and no
    # query/key gradient; a zero query row (D_t = 0, eps = 0) passes nothing
    T, d, dv = 6, 3, 2
    q, k, v, do = _data(T, d, dv, seed=9)
    g = np.zeros_like(do)
    g[0] = do[0]
    dq, dk, dv_ = O.prefill_backward(q, k, v, g)
    np.testing.assert_allclose(dv_[0], do[0], rtol=1e-14)
    np.testing.assert_allclose(dv_[1:], 0.0, atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    q[3] = 0.0
    dq, dk, dv_ = O.prefill_backward(q, k, v, do)
    assert np.all(dq[3] == 0.0)
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv_))


@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_row_form_matches_full(eps):
    T, d, dv = 300, 16, 8
    q, k, v, do = _data(T, d, dv, seed=21)
    dq, dk, dv_ = O.prefill_backward(q, k, v, do, eps=eps)
    rows = [0, 1, 37, 150, 299]
    rq, rk, rv = O.prefill_backward_rows(q, k, v, do, rows, rows, eps=eps, chunk=64)
    np.testing.assert_allclose(rq, dq[rows], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(rk, dk[rows], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(rv, dv_[rows], rtol=1e-9, atol=1e-12)

