"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a dropped sqrt(2), a dropped diagonal, a read-before-update,
a transposed intra-chunk operand, an unnormalised prediction, a reversed
selection, a fold of the kept pairs, a gradient without its centering term,
swapped query and key gradients."""
import functools

import numpy as np
import pytest

import oracle as O
import oracle.kla_oracle as K
from tests import test_oracle_backward as TB
from tests import test_oracle_hybrid as TH
from tests import test_oracle_phi_prefill as TP
from tests import test_oracle_sre_select as TS


def _phi_no_sqrt2(x):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    return np.stack([x[..., i] * x[..., j] for i in range(d) for j in range(i, d)], axis=-1)


def _chunked_strict_lower(q, k, v, chunk=256, H0=None, s0=None, eps=0.0, return_parts=False):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    T, d = q.shape
    H = np.zeros((O.phi_dim(d), v.shape[1]))
    s = np.zeros(O.phi_dim(d))
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        Q, Kc, V = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk]
        S = Q @ Kc.T
        A = np.tril(S * S, k=-1)  # planted: diagonal dropped
        num = A @ V + O.phi(Q) @ H
        den = A.sum(1) + O.phi(Q) @ s
        o[c0:c0 + chunk] = K._safe_div(num, den)
        H += O.phi(Kc).T @ V
        s += O.phi(Kc).sum(0)
    return o, H, s


def _chunked_transposed(q, k, v, chunk=256, H0=None, s0=None, eps=0.0, return_parts=False):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    T, d = q.shape
    H = np.zeros((O.phi_dim(d), v.shape[1]))
    s = np.zeros(O.phi_dim(d))
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        Q, Kc, V = q[c0:c0 + chunk], k[c0:c0 + chunk], v[c0:c0 + chunk]
        S = Kc @ Q.T  # planted: keys against queries
        A = np.tril(S * S)
        num = A @ V + O.phi(Q) @ H
        den = A.sum(1) + O.phi(Q) @ s
        o[c0:c0 + chunk] = K._safe_div(num, den)
        H += O.phi(Kc).T @ V
        s += O.phi(Kc).sum(0)
    return o, H, s


def _decode_read_first(H, s, q, k, v, eps=0.0):
    fq = O.phi(q)
    den = fq @ s + eps
    o = (fq @ H) / den if den else np.zeros(np.shape(H)[1])  # planted: read before update
    fk = O.phi(k)
    return o, H + np.outer(fk, v), s + fk


def _sre_unnormalised(H, s, k, v, eps=0.0):
    pred = O.phi(k) @ H  # planted: no division by phi(k).s
    return np.sum((pred - v) ** 2, axis=-1)


def _select_ascending(scores, m, ids=None):
    ids = np.arange(len(scores)) if ids is None else np.asarray(ids)
    return np.lexsort((ids, np.asarray(scores)))[:m]  # planted: lowest first


def _backward_no_centering(q, k, v, do, eps=0.0):
    # planted: forgets the -c_t term of the denominator's derivative
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    S = np.tril(q @ k.T)
    W = S * S
    D = W.sum(axis=1) + eps
    dv = (W / D[:, None]).T @ do
    dS = np.tril(2.0 * S * (do @ v.T) / D[:, None])
    return dS @ k, dS.T @ q, dv


def _backward_transposed(q, k, v, do, eps=0.0):
    # planted: query and key gradients swapped
    dq, dk, dv = REAL_BACKWARD(q, k, v, do, eps=eps)
    return dk, dq, dv


REAL_BACKWARD = O.prefill_backward

CASES = [
    ("phi", _phi_no_sqrt2, [TP.test_phi_golden, TP.test_phi_random_float_identity]),
    ("prefill_chunked", _chunked_strict_lower, [TP.test_first_token_returns_its_value]),
    ("prefill_chunked_transposed", _chunked_transposed,
     [functools.partial(TP.test_forms_agree_on_small_integers, 7),
      functools.partial(TP.test_three_forms_agree, 3, 57, 32)]),
    ("decode_step", _decode_read_first, [TS.test_decode_step_matches_definition_cases]),
    ("sre", _sre_unnormalised, [TS.test_sre_golden]),
    ("select_topk", _select_ascending, [TS.test_select_topk_order_against_python_sort]),
    ("prefill_backward", _backward_no_centering, [TB.test_homogeneity_identities]),
    ("prefill_backward_transposed", _backward_transposed,
     [functools.partial(TB.test_gradients_match_finite_differences, 7, 3, 2, 0.0)]),
]


@pytest.mark.parametrize("name,bad,pins", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_planted_mistake(monkeypatch, name, bad, pins):
    name = name.replace("_transposed", "")
    monkeypatch.setattr(O, name, bad)
    monkeypatch.setattr(K, name, bad)
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {name}"


def test_hybrid_pin_catches_fold_of_kept_pairs(monkeypatch):
    real_select = K.select_topk

    def select_complement(scores, m, ids=None):
        # planted: keep the lowest-score pairs (fold the hard ones)
        order = real_select(-np.asarray(scores), len(scores), ids)
        return order[:m]

    monkeypatch.setattr(K, "select_topk", select_complement)
    with pytest.raises(AssertionError):
        TH.test_refresh_chain_against_token_by_token_enumeration(3, 16, 4, 8)


# ---- multi-factor lifts (KATA-Mg / KATA-Sigma-g)

from tests import test_oracle_factors as TF  # noqa: E402

_real_factor_weights = K.factor_weights
_real_phi_factors = K.phi_factors


def _weights_no_cross_terms(q, k, g, kind):
    return _real_factor_weights(q, k, g, "concat")  # planted: Sigma-g loses q_i . k_j, i != j


def _weights_square_of_sum(q, k, g, kind):
    if kind == "concat":  # planted: (sum_i q_i . k_i)^2, the rank-one kernel again
        qs, ks = K._factors(np.asarray(q, np.float64), g), K._factors(np.asarray(k, np.float64), g)
        return sum(a @ b.T for a, b in zip(qs, ks)) ** 2
    return _real_factor_weights(q, k, g, kind)


def _phi_factors_no_sqrt2(x, g, kind):
    if kind != "sum":
        return _real_phi_factors(x, g, kind)
    parts = K._factors(np.asarray(x, np.float64), g)
    p = parts[0].shape[-1]
    M = sum(u[..., :, None] * u[..., None, :] for u in parts)
    i, j = np.triu_indices(p)
    return M[..., i, j]  # planted: off-diagonal sqrt(2) dropped


@pytest.mark.parametrize("name,bad", [("factor_weights", _weights_no_cross_terms),
                                      ("factor_weights", _weights_square_of_sum),
                                      ("phi_factors", _phi_factors_no_sqrt2)],
                         ids=["sum_without_cross_terms", "concat_as_square_of_sum", "sum_lift_without_sqrt2"])
def test_factor_pins_catch_planted_mistake(monkeypatch, name, bad):
    monkeypatch.setattr(O, name, bad)
    monkeypatch.setattr(K, name, bad)
    pins = [TF.test_worked_integer_example,
            functools.partial(TF.test_state_form_equals_closed_form, 2, "sum"),
            functools.partial(TF.test_state_form_equals_closed_form, 2, "concat")]
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {name}"
