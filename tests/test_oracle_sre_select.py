"""Pins for the oracle's decode step, self-recall error, selection and the
decode + selection chain (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _state(keys, values):
    D = O.phi_dim(keys.shape[1])
    fk = O.phi(keys)
    return fk.T @ values, fk.sum(axis=0)


def test_sre_golden():
    g = json.load(open(os.path.join(GOLD, "sre_small.json")))
    for c in g["cases"]:
        pk, pv, ck, cv = (np.array(c[x], np.float64) for x in ("pairs_k", "pairs_v", "cand_k", "cand_v"))
        H, s = _state(pk, pv)
        np.testing.assert_allclose(O.sre(H, s, ck, cv), c["sre"], rtol=1e-14)
        np.testing.assert_allclose(O.sre_bruteforce(pk, pv, ck, cv), c["sre"], rtol=1e-14)


@pytest.mark.parametrize("d", [3, 16, 64])
def test_sre_zero_for_signed_basis_keys(d):
    # phi(e_i).phi(e_j) = delta_ij: each stored key recalls its own value
    # exactly, in any precision.
    rng = np.random.default_rng(d)
    m = min(d, 12)
    idx = rng.choice(d, m, replace=False)
    keys = np.eye(d)[idx] * rng.choice([-1.0, 1.0], m)[:, None]
    vals = rng.standard_normal((m, 5))
    H, s = _state(keys, vals)
    assert np.all(O.sre(H, s, keys, vals) == 0.0)


@pytest.mark.parametrize("d", [4, 16, 64])
def test_sre_near_zero_for_orthonormal_keys(d):
    rng = np.random.default_rng(50 + d)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Q[: min(d, 20)]
    vals = rng.standard_normal((len(keys), 7))
    H, s = _state(keys, vals)
    sc = O.sre(H, s, keys, vals)
    assert np.all(sc <= 1e-20), sc.max()


def test_sre_state_form_equals_bruteforce():
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((200, 8))
    vals = rng.standard_normal((200, 6))
    H, s = _state(keys, vals)
    ck = rng.standard_normal((30, 8))
    cv = rng.standard_normal((30, 6))
    np.testing.assert_allclose(O.sre(H, s, ck, cv), O.sre_bruteforce(keys, vals, ck, cv), rtol=1e-12)


def test_sre_empty_state_and_key_scale():
    rng = np.random.default_rng(12)
    d, dv = 6, 4
    D = O.phi_dim(d)
    ck = rng.standard_normal((5, d))
    cv = rng.standard_normal((5, dv))
    np.testing.assert_allclose(O.sre(np.zeros((D, dv)), np.zeros(D), ck, cv), np.sum(cv ** 2, axis=1))
    keys = rng.standard_normal((40, d))
    vals = rng.standard_normal((40, dv))
    H, s = _state(keys, vals)
    np.testing.assert_allclose(O.sre(H, s, 2.5 * ck, cv), O.sre(H, s, ck, cv), rtol=1e-12)
    # all stored keys equal: every candidate (not orthogonal to it) predicts
    # the mean stored value
    Hm, sm = _state(np.tile(keys[0], (40, 1)), vals)
    want = np.sum((vals.mean(axis=0) - cv) ** 2, axis=1)
    np.testing.assert_allclose(O.sre(Hm, sm, ck, cv), want, rtol=1e-12)


def test_decode_step_matches_definition_cases():
    # first token into an empty state returns its own value; the update comes
    # before the readout.
    rng = np.random.default_rng(13)
    d, dv = 5, 3
    D = O.phi_dim(d)
    q, k, v = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(dv)
    o, H, s = O.decode_step(np.zeros((D, dv)), np.zeros(D), q, k, v)
    np.testing.assert_allclose(o, v, rtol=1e-14)
    np.testing.assert_allclose(s, O.phi(k), rtol=0)


def test_select_topk_order_against_python_sort():
    rng = np.random.default_rng(14)
    for _ in range(50):
        n = int(rng.integers(1, 80))
        sc = rng.integers(0, 6, n).astype(float)  # many ties
        m = int(rng.integers(0, n + 1))
        want = sorted(range(n), key=lambda i: (-sc[i], i))[:m]
        assert list(O.select_topk(sc, m)) == want
        ids = rng.permutation(1000)[:n]
        want_ids = sorted(range(n), key=lambda i: (-sc[i], ids[i]))[:m]
        assert list(O.select_topk(sc, m, ids=ids)) == want_ids


def test_near_tie_rule():
    sc = np.array([5.0, 4.0, 3.0, 2.0])
    assert O.near_tie_ok(sc, [0, 1], 2)
    assert O.near_tie_ok(sc, [1, 0], 2)
    assert not O.near_tie_ok(sc, [0, 2], 2)
    tie = np.array([5.0, 3.0, 3.0 * (1 - 1e-7), 1.0])
    assert O.near_tie_ok(tie, [0, 1], 2)
    assert O.near_tie_ok(tie, [0, 2], 2)
    assert not O.near_tie_ok(tie, [1, 2], 2)  # the clear winner 0 must be kept
    assert not O.near_tie_ok(tie, [0, 3], 2)


def test_decode_chain_small_hand_checkable():
    # 2 head-states, 8 steps, d = 4, top 3 of 3 cached + 5 fresh.
    rng = np.random.default_rng(15)
    d, dv, S, K, F = 4, 3, 8, 3, 5
    D = O.phi_dim(d)
    for n in range(2):
        pk = rng.standard_normal((20, d)) / 2
        pv = rng.standard_normal((20, dv))
        H0, s0 = _state(pk, pv)
        q = rng.standard_normal((S, d)) / 2
        k = rng.standard_normal((S, d)) / 2
        v = rng.standard_normal((S, dv))
        fk = rng.standard_normal((S, F, d)) / 2
        fv = rng.standard_normal((S, F, dv))
        ck = rng.standard_normal((K, d)) / 2
        cv = rng.standard_normal((K, dv))
        r = O.decode_sre_chain(H0, s0, q, k, v, fk, fv, ck, cv, K)
        # step 0 scores, by brute force over the prefix pairs plus the new token
        allk = np.concatenate([pk, k[:1]])
        allv = np.concatenate([pv, v[:1]])
        cand_k = np.concatenate([ck, fk[0]])
        cand_v = np.concatenate([cv, fv[0]])
        np.testing.assert_allclose(r["scores"][0], O.sre_bruteforce(allk, allv, cand_k, cand_v), rtol=1e-11)
        # outputs equal a prefill over prefix + step tokens (candidates never
        # touch the state)
        o_ref = O.prefill_recurrent(np.concatenate([pk, q]), np.concatenate([pk, k]),
                                    np.concatenate([pv, v]))
        np.testing.assert_allclose(r["o"], o_ref[0][20:], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(r["H"], o_ref[1], rtol=1e-12, atol=1e-12)
        # the cache follows the selection, step by step
        cache_k = ck.copy()
        for tau in range(S):
            cand = np.concatenate([cache_k, fk[tau]])
            sel = r["sel"][tau]
            assert list(sel) == sorted(range(K + F), key=lambda i: (-r["scores"][tau][i], i))[:K]
            cache_k = cand[sel]
        np.testing.assert_allclose(r["cache_k"], cache_k)
