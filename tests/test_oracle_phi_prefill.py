"""Pins for the oracle's lift and its three prefill forms (CPU only).

Each pin rests on something other than the oracle's own formula: the
hand-derived fixtures in tests/golden/, exact integer arithmetic, closed
forms (cumulative means, one-hot keys, d = 1), and identities of the method
(convex output gate of KATA §2.1, resumability of the fixed-size state).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _over(d):
    return np.asarray(d["exact"], np.float64) + math.sqrt(2.0) * np.asarray(d["times_sqrt2"], np.float64)


# ---------------------------------------------------------------- lift

def test_phi_golden():
    g = json.load(open(os.path.join(GOLD, "phi_small.json")))
    for c in g["cases"]:
        got = O.phi(np.array(c["x"], np.float64))
        np.testing.assert_allclose(got, _over(c["phi_over"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("d", [1, 2, 3, 5, 16, 32, 64])
def test_phi_dim_and_order(d):
    pairs = O.phi_pairs(d)
    assert len(pairs) == O.phi_dim(d) == d * (d + 1) // 2
    for f, (i, j) in enumerate(pairs):
        assert f == i * d - i * (i - 1) // 2 + (j - i)
        assert i <= j


@pytest.mark.parametrize("d", [1, 2, 3, 7, 16, 64])
def test_phi_squares_inner_product_integers(d):
    # phi(x).phi(y) = (x.y)^2, checked against exact integer arithmetic.
    rng = np.random.default_rng(100 + d)
    for _ in range(20):
        x = rng.integers(-3, 4, size=d)
        y = rng.integers(-3, 4, size=d)
        exact = int(sum(int(a) * int(b) for a, b in zip(x, y))) ** 2
        got = float(O.phi(x.astype(np.float64)) @ O.phi(y.astype(np.float64)))
        assert abs(got - exact) <= 1e-13 * max(1.0, exact)
        # and the feature norm is the squared vector norm
        nx = int(sum(int(a) ** 2 for a in x))
        assert abs(float(O.phi(x.astype(float)) @ O.phi(x.astype(float))) - nx * nx) <= 1e-13 * max(1, nx * nx)


def test_phi_random_float_identity():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, 64))
    y = rng.standard_normal((50, 64))
    lhs = np.sum(O.phi(x) * O.phi(y), axis=1)
    rhs = np.sum(x * y, axis=1) ** 2
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- prefill

def test_prefill_golden():
    g = json.load(open(os.path.join(GOLD, "prefill_small.json")))
    for c in g["cases"]:
        q, k, v = (np.array(c[x], np.float64) for x in ("q", "k", "v"))
        for fn in (lambda: O.prefill_bruteforce(q, k, v),
                   lambda: O.prefill_recurrent(q, k, v)[0],
                   lambda: O.prefill_chunked(q, k, v, chunk=2)[0]):
            np.testing.assert_allclose(fn(), np.array(c["o"], np.float64), rtol=0, atol=1e-14)
        _, H, s = O.prefill_chunked(q, k, v, chunk=2)
        if "H" in c:
            np.testing.assert_allclose(H, np.array(c["H"], np.float64), atol=1e-14)
            np.testing.assert_allclose(s, np.array(c["s"], np.float64), atol=1e-14)
        else:
            np.testing.assert_allclose(H, _over(c["H_over"]), atol=1e-14)
            np.testing.assert_allclose(s, _over(c["s_over"]), atol=1e-14)


def test_bruteforce_all_equal_keys_is_cumulative_mean():
    # Equal weights for every past token: o_t is the running mean of v.
    rng = np.random.default_rng(1)
    T, d = 40, 5
    key = rng.standard_normal(d)
    k = np.tile(key, (T, 1))
    q = rng.standard_normal((T, d))
    v = rng.standard_normal((T, 3))
    want = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(O.prefill_bruteforce(q, k, v), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.prefill_chunked(q, k, v, chunk=7)[0], want, rtol=1e-12, atol=1e-12)


def test_bruteforce_one_hot_keys_select_matching_tokens():
    # q_t = e_a, k_i = e_b: weight 1 iff a == b and i <= t; the output is the
    # mean of the matching past values (checks causality and operand order).
    rng = np.random.default_rng(2)
    T, d = 60, 4
    a = rng.integers(0, d, T)
    b = rng.integers(0, d, T)
    b[0] = a[0]
    q = np.eye(d)[a]
    k = np.eye(d)[b]
    v = rng.standard_normal((T, 2))
    want = np.zeros((T, 2))
    for t in range(T):
        idx = [i for i in range(t + 1) if b[i] == a[t]]
        want[t] = v[idx].mean(axis=0) if idx else 0.0
    for got in (O.prefill_bruteforce(q, k, v), O.prefill_recurrent(q, k, v)[0],
                O.prefill_chunked(q, k, v, chunk=9)[0]):
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("d,T", [(2, 30), (3, 57), (16, 256)])
@pytest.mark.parametrize("chunk", [1, 7, 32, None])
def test_three_forms_agree(d, T, chunk):
    rng = np.random.default_rng(d * 1000 + T)
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, 4))
    ob, nb, db = O.prefill_bruteforce(q, k, v, return_parts=True)
    orr, Hr, sr, nr, dr = O.prefill_recurrent(q, k, v, return_parts=True)
    oc, Hc, sc, nc, dc = O.prefill_chunked(q, k, v, chunk=chunk or T, return_parts=True)
    for x in (orr, oc):
        np.testing.assert_allclose(x, ob, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Hc, Hr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sc, sr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dc, db, rtol=1e-12)
    np.testing.assert_allclose(dr, db, rtol=1e-12)


@pytest.mark.parametrize("chunk", [1, 7, 32, 300])
def test_forms_agree_on_small_integers(chunk):
    # numerators and denominators are integers; the sqrt(2) scaling on both
    # sides leaves them exact to a few ulps.
    rng = np.random.default_rng(9)
    T, d = 300, 3
    q = rng.integers(-3, 4, (T, d)).astype(float)
    k = rng.integers(-3, 4, (T, d)).astype(float)
    v = rng.integers(-3, 4, (T, 2)).astype(float)
    _, nb, db = O.prefill_bruteforce(q, k, v, return_parts=True)
    # exact integer reference for the denominators
    dint = np.array([sum(int(np.dot(q[t].astype(int), k[i].astype(int))) ** 2 for i in range(t + 1))
                     for t in range(T)], dtype=np.float64)
    np.testing.assert_array_equal(db, dint)
    _, _, _, nr, dr = O.prefill_recurrent(q, k, v, return_parts=True)
    _, _, _, nc, dc = O.prefill_chunked(q, k, v, chunk=chunk, return_parts=True)
    for n_, d_ in ((nr, dr), (nc, dc)):
        np.testing.assert_allclose(d_, dint, rtol=1e-14)
        np.testing.assert_allclose(n_, nb, rtol=1e-14, atol=1e-8)


def test_first_token_returns_its_value():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((5, 8))
    v = rng.standard_normal((5, 8))
    for o in (O.prefill_bruteforce(q, k, v), O.prefill_chunked(q, k, v, 3)[0]):
        np.testing.assert_allclose(o[0], v[0], rtol=1e-14)


def test_convex_output_gate_identity_and_bounds():
    # KATA §2.1: the denominator acts as a parameter-free convex gate between
    # the previous readout and the current value:
    # o_t = (1 - g_t) ohat_t + g_t v_t, g_t = (q_t.k_t)^2 / phi(q_t).s_t.
    rng = np.random.default_rng(4)
    T, d, dv = 50, 6, 3
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, dv))
    o, _, _ = O.prefill_recurrent(q, k, v)
    D = O.phi_dim(d)
    H = np.zeros((D, dv))
    s = np.zeros(D)
    for t in range(T):
        fq = O.phi(q[t])
        den_prev = fq @ s
        ohat = (fq @ H) / den_prev if den_prev > 0 else np.zeros(dv)
        fk = O.phi(k[t])
        s += fk
        H += np.outer(fk, v[t])
        g = float(np.dot(q[t], k[t]) ** 2 / (fq @ s))
        assert -1e-15 <= g <= 1 + 1e-15
        np.testing.assert_allclose(o[t], (1 - g) * ohat + g * v[t], rtol=1e-10, atol=1e-12)
        lo = v[: t + 1].min(axis=0)
        hi = v[: t + 1].max(axis=0)
        assert np.all(o[t] >= lo - 1e-12) and np.all(o[t] <= hi + 1e-12)


def test_invariances():
    rng = np.random.default_rng(5)
    T, d = 40, 5
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, 2))
    o = O.prefill_chunked(q, k, v, 8)[0]
    c = rng.uniform(0.5, 2.0, T)
    np.testing.assert_allclose(O.prefill_chunked(q * c[:, None], k, v, 8)[0], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(O.prefill_chunked(q, 3.0 * k, v, 8)[0], o, rtol=1e-11, atol=1e-12)
    # a common rotation of q and k leaves every (q.k)^2 unchanged
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    np.testing.assert_allclose(O.prefill_chunked(q @ Q, k @ Q, v, 8)[0], o, rtol=1e-10, atol=1e-11)


def test_resume_and_decode_equal_prefill():
    rng = np.random.default_rng(6)
    T1, T2, d = 37, 29, 4
    q = rng.standard_normal((T1 + T2, d))
    k = rng.standard_normal((T1 + T2, d))
    v = rng.standard_normal((T1 + T2, 3))
    o, H, s = O.prefill_chunked(q, k, v, 8)
    o1, H1, s1 = O.prefill_chunked(q[:T1], k[:T1], v[:T1], 8)
    o2, H2, s2 = O.prefill_chunked(q[T1:], k[T1:], v[T1:], 5, H0=H1, s0=s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(H2, H, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2, s, rtol=1e-12, atol=1e-12)
    D = O.phi_dim(d)
    Hd, sd = np.zeros((D, 3)), np.zeros(D)
    for t in range(T1 + T2):
        ot, Hd, sd = O.decode_step(Hd, sd, q[t], k[t], v[t])
        np.testing.assert_allclose(ot, o[t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Hd, H, rtol=1e-12, atol=1e-12)


def test_zero_denominator_gives_zero_and_eps():
    q = np.zeros((3, 2))
    k = np.ones((3, 2))
    v = np.ones((3, 2))
    assert np.all(O.prefill_chunked(q, k, v, 2)[0] == 0)
    assert np.all(O.prefill_bruteforce(q, k, v) == 0)
    # eps enters every denominator once
    q = np.ones((2, 1))
    k = np.ones((2, 1))
    v = np.array([[2.0], [4.0]])
    o = O.prefill_chunked(q, k, v, 2, eps=1.0)[0]
    np.testing.assert_allclose(o[:, 0], [2.0 / 2.0, 6.0 / 3.0])


def test_bruteforce_rows_match_full():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((70, 6))
    k = rng.standard_normal((70, 6))
    v = rng.standard_normal((70, 3))
    rows = [0, 5, 31, 69]
    np.testing.assert_allclose(O.prefill_bruteforce_rows(q, k, v, rows),
                               O.prefill_bruteforce(q, k, v)[rows], rtol=1e-13)
