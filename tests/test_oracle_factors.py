"""Pins for the oracle's multi-factor lifts (KATA-Mg "concat", KATA-Sigma-g
"sum"; CPU only).

They are pinned by a worked integer example done by hand, by the special
cases g = 1 (the rank-one lift) and g = d (closed forms), by the symmetries
the two definitions imply (factor permutations, factor sign flips), and by
the equality of two independent forms of the prefill (closed-form weights vs
the fixed-size state).
"""
import numpy as np
import pytest

import oracle as O


def test_worked_integer_example():
    # d = 4, g = 2: q = ([1, 2], [3, 4]), k = ([2, 0], [1, 1])
    # q1.k1 = 2, q2.k2 = 7, q1.k2 = 3, q2.k1 = 6
    q = np.array([1.0, 2.0, 3.0, 4.0])
    k = np.array([2.0, 0.0, 1.0, 1.0])
    cat = O.phi_factors(q, 2, "concat") @ O.phi_factors(k, 2, "concat")
    summ = O.phi_factors(q, 2, "sum") @ O.phi_factors(k, 2, "sum")
    assert cat == pytest.approx(4.0 + 49.0, rel=1e-14)
    assert summ == pytest.approx(4.0 + 49.0 + 9.0 + 36.0, rel=1e-14)
    W = O.factor_weights(q[None], k[None], 2, "concat")
    assert W[0, 0] == pytest.approx(53.0, rel=1e-14)
    assert O.factor_weights(q[None], k[None], 2, "sum")[0, 0] == pytest.approx(98.0, rel=1e-14)


def test_feature_dimensions():
    x = np.ones((3, 64))
    assert O.phi_factors(x, 1, "concat").shape == (3, 2080)
    assert O.phi_factors(x, 2, "concat").shape == (3, 2 * 528)
    assert O.phi_factors(x, 4, "concat").shape == (3, 4 * 136)
    assert O.phi_factors(x, 2, "sum").shape == (3, 528)
    assert O.phi_factors(x, 4, "sum").shape == (3, 136)
    with pytest.raises(ValueError):
        O.phi_factors(x, 3, "sum")


@pytest.mark.parametrize("kind", O.FACTOR_KINDS)
def test_one_factor_is_the_rank_one_lift(kind):
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((40, 8)), rng.standard_normal((40, 8)), rng.standard_normal((40, 5))
    np.testing.assert_allclose(O.phi_factors(q, 1, kind), O.phi(q), rtol=1e-15, atol=0)
    np.testing.assert_allclose(O.prefill_factors_bruteforce(q, k, v, 1, kind, eps=0.1),
                               O.prefill_bruteforce(q, k, v, eps=0.1), rtol=1e-13, atol=1e-15)


def test_one_dimensional_factors_closed_forms():
    # g = d: concat gives sum_a q_a^2 k_a^2; sum gives |q|^2 |k|^2, so the
    # output no longer depends on the query: o_t = sum_i |k_i|^2 v_i / sum_i |k_i|^2
    rng = np.random.default_rng(4)
    T, d = 30, 6
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, 3))
    np.testing.assert_allclose(O.factor_weights(q, k, d, "concat"), (q * q) @ (k * k).T, rtol=1e-13)
    o = O.prefill_factors_bruteforce(q, k, v, d, "sum")
    nk = np.sum(k * k, axis=1)
    ref = np.cumsum(nk[:, None] * v, axis=0) / np.cumsum(nk)[:, None]
    np.testing.assert_allclose(o, ref, rtol=1e-12)


def test_factor_symmetries():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((7, 12)), rng.standard_normal((9, 12))
    perm = lambda x, order: np.concatenate([x[:, 4 * i:4 * i + 4] for i in order], axis=1)
    flip = np.repeat([1.0, -1.0, 1.0], 4)
    Wc, Ws = O.factor_weights(q, k, 3, "concat"), O.factor_weights(q, k, 3, "sum")
    # concat: the same factor permutation on both sides; any factor's sign
    np.testing.assert_allclose(O.factor_weights(perm(q, [2, 0, 1]), perm(k, [2, 0, 1]), 3, "concat"), Wc, rtol=1e-13)
    np.testing.assert_allclose(O.factor_weights(q * flip, k, 3, "concat"), Wc, rtol=1e-13)
    # sum: independent permutations of the query's and the key's factors
    np.testing.assert_allclose(O.factor_weights(perm(q, [1, 2, 0]), perm(k, [2, 1, 0]), 3, "sum"), Ws, rtol=1e-13)
    np.testing.assert_allclose(O.factor_weights(q, k * flip, 3, "sum"), Ws, rtol=1e-13)
    # and the two differ once the factors interact
    assert np.max(np.abs(Ws - Wc)) > 1e-3


@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("kind", O.FACTOR_KINDS)
def test_state_form_equals_closed_form(g, kind):
    # the feature map's inner product equals the closed-form weight, so the
    # fixed-size recurrence reproduces the O(T^2) definition
    rng = np.random.default_rng(10 + g)
    T, d = 50, 16
    q, k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.standard_normal((T, 4))
    np.testing.assert_allclose(O.phi_factors(q, g, kind) @ O.phi_factors(k, g, kind).T,
                               O.factor_weights(q, k, g, kind), rtol=1e-12, atol=1e-12)
    o_state, H, s = O.prefill_factors_recurrent(q, k, v, g, kind, eps=0.05)
    o_bf = O.prefill_factors_bruteforce(q, k, v, g, kind, eps=0.05)
    np.testing.assert_allclose(o_state, o_bf, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s, O.phi_factors(k, g, kind).sum(axis=0), rtol=1e-12)
