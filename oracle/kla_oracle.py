"""Float64 CPU oracle for causal kernelized linear attention.

TEST INFRASTRUCTURE. Only the tests, the package's ``smoke()`` check and the
benchmark's CPU-baseline leg may import or call this module. It imports
nothing from the GPU library or its binding, and the GPU library shares no
code with it. Speed is not a goal: every function is the plain definition or
the plain algorithm, in float64, with NumPy matrix products as the only
library primitive.

Pages cited (titles and sections of the pages themselves):
  KATA = "Kernelized Linear Attention: Breaking the Capacity Wall with
         Symmetric Cones" (gist.science/pt/paper/2607.17419);
  LoLA = "LoLA: Low-Rank Linear Attention with Sparse Caching", Portuguese
         technical summary (gist.science/pt/paper/2505.23666).

Readings where the pages are silent (each one is listed with its reason in
the design notes of the repository):
  * phi order: upper triangle, row-major, f(i, j) = i*d - i*(i-1)/2 + (j-i),
    off-diagonal coordinates scaled by sqrt(2); this is the isometric
    vectorisation of the symmetric matrix x x^T, so phi(x).phi(y) equals the
    Frobenius product <x x^T, y y^T> = (x.y)^2.
  * no projection before the lift, no temperature on (q.k)^2;
  * causal sums include the current token (i <= t); a decode step updates
    the state before it reads it out;
  * eps is added to every denominator; a zero denominator gives a zero
    output (and a zero self-recall prediction);
  * top-k order: (score descending, index ascending);
  * hybrid: block-aligned eviction frontier, one joint normalisation of the
    window, cache and linear terms, self-recall scored against the state
    before that refresh's fold.

Parity pins: every function here is pinned by a test under tests/ against a
closed form, an identity of the mathematics, a special case that reduces to
a textbook routine, or brute force on tiny inputs. The hybrid conventions
(eviction frontier, joint normalisation, tie order, empty-state prediction)
are readings of the LoLA page and are pinned only through the special cases
and a brute-force re-enumeration of the refresh chain.
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import numpy as np

SQRT2 = math.sqrt(2.0)


# ----------------------------------------------------------------------------
# Feature lift
# ----------------------------------------------------------------------------

def phi_dim(d: int) -> int:
    """D = d(d+1)/2, the dimension of the symmetric-matrix feature."""
    return d * (d + 1) // 2


def phi_pairs(d: int):
    """Coordinate order of phi: list of (i, j), i <= j, upper triangle row-major."""
    return [(i, j) for i in range(d) for j in range(i, d)]


def phi(x: np.ndarray) -> np.ndarray:
    """Rank-one PSD lift psi(u) = u u^T of KATA §2.2, vectorised.

    The page's lift squares the raw inner product, <u_i, u_j>^2. Written as
    a vector: x_i^2 on the diagonal and sqrt(2) x_i x_j above it, so that
    phi(x) . phi(y) = sum_i x_i^2 y_i^2 + sum_{i<j} 2 x_i x_j y_i y_j
                    = (x . y)^2.
    x: [..., d] -> [..., d(d+1)/2], float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pairs = phi_pairs(d)
    i = np.array([a for a, _ in pairs], dtype=np.intp)
    j = np.array([b for _, b in pairs], dtype=np.intp)
    c = np.where(i == j, 1.0, SQRT2)
    # (c_f * x_i) * x_j: 1 * x_i * x_i on the diagonal, sqrt(2) * x_i * x_j above it
    return (c * x[..., i]) * x[..., j]


def _safe_div(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """num / den row-wise; rows whose denominator is exactly 0 give 0."""
    den = np.asarray(den, dtype=np.float64)
    out = np.zeros(np.broadcast_shapes(np.shape(num)), dtype=np.float64)
    nz = den != 0
    if np.ndim(num) == np.ndim(den) + 1:
        out[nz] = num[nz] / den[nz][..., None]
    else:
        out[nz] = num[nz] / den[nz]
    return out


# ----------------------------------------------------------------------------
# Multi-factor PSD lifts (KATA §2.3, "Variantes": KATA-Mg with several PSD
# factors and KATA-Sigma-g with summed PSD factors). The page names the two
# variants and their purpose (trading state size against packing) but not how
# the factors are formed. Reading taken here: the d dimensions of q and k are
# split into g equal factors x_1 .. x_g of p = d / g dimensions each, and
#   Mg:  phi(x) = [psi(x_1), ..., psi(x_g)], the rank-one lifts concatenated
#        (g p(p+1)/2 features), so phi(q).phi(k) = sum_i (q_i . k_i)^2;
#   Sg:  phi(x) = psi-vectorisation of sum_i x_i x_i^T, the factors' outer
#        products summed before the lift (p(p+1)/2 features), so
#        phi(q).phi(k) = <sum_i q_i q_i^T, sum_j k_j k_j^T>_F
#                      = sum_{i,j} (q_i . k_j)^2.
# With g = 1 both are the rank-one lift above.
# ----------------------------------------------------------------------------

FACTOR_KINDS = ("concat", "sum")


def _factors(x: np.ndarray, g: int):
    d = x.shape[-1]
    if g < 1 or d % g:
        raise ValueError(f"g = {g} must divide d = {d}")
    p = d // g
    return [x[..., i * p:(i + 1) * p] for i in range(g)]


def phi_factors(x, g: int, kind: str) -> np.ndarray:
    """The feature vector of the KATA-Mg ("concat") or KATA-Sigma-g ("sum")
    variant; x: [..., d] -> [..., g p(p+1)/2] or [..., p(p+1)/2]."""
    x = np.asarray(x, dtype=np.float64)
    parts = _factors(x, g)
    if kind == "concat":
        return np.concatenate([phi(u) for u in parts], axis=-1)
    if kind != "sum":
        raise ValueError(kind)
    p = parts[0].shape[-1]
    M = sum(u[..., :, None] * u[..., None, :] for u in parts)      # sum_i x_i x_i^T
    i, j = np.triu_indices(p)
    return np.where(i == j, 1.0, SQRT2) * M[..., i, j]


def factor_weights(q, k, g: int, kind: str) -> np.ndarray:
    """Closed-form kernel between every query and key row: W[t, s] =
    sum_i (q_t,i . k_s,i)^2 (concat) or sum_{i,j} (q_t,i . k_s,j)^2 (sum)."""
    qs, ks = _factors(np.asarray(q, np.float64), g), _factors(np.asarray(k, np.float64), g)
    if kind == "concat":
        return sum((a @ b.T) ** 2 for a, b in zip(qs, ks))
    if kind != "sum":
        raise ValueError(kind)
    return sum((a @ b.T) ** 2 for a in qs for b in ks)


def prefill_factors_bruteforce(q, k, v, g: int, kind: str, eps: float = 0.0, return_parts: bool = False):
    """Causal attention with the variant's closed-form weights, normalised
    over i <= t (the O(T^2) definition, as prefill_bruteforce for g = 1)."""
    W = np.tril(factor_weights(q, k, g, kind))
    v = np.asarray(v, np.float64)
    num = W @ v
    den = W.sum(axis=1) + eps
    o = _safe_div(num, den)
    return (o, num, den) if return_parts else o


def prefill_factors_recurrent(q, k, v, g: int, kind: str, eps: float = 0.0):
    """The same outputs through the variant's fixed-size state:
    H += phi(k_t) v_t^T, s += phi(k_t), o_t = phi(q_t)^T H / (phi(q_t)^T s + eps).
    Returns o [T, dv], H [D_g, dv], s [D_g]."""
    fq, fk = phi_factors(q, g, kind), phi_factors(k, g, kind)
    v = np.asarray(v, np.float64)
    H = np.zeros((fk.shape[1], v.shape[1]))
    s = np.zeros(fk.shape[1])
    o = np.zeros_like(v)
    for t in range(v.shape[0]):
        H += np.outer(fk[t], v[t])
        s += fk[t]
        den = fq[t] @ s + eps
        o[t] = fq[t] @ H / den if den != 0 else 0.0
    return o, H, s


# ----------------------------------------------------------------------------
# Prefill: three forms of the same result (one (b, h) head; q,k [T,d], v [T,dv])
# ----------------------------------------------------------------------------

def prefill_bruteforce(q, k, v, eps: float = 0.0, return_parts: bool = False):
    """Causal attention with weights (q_t.k_i)^2 normalised over i <= t.

    This is the plain O(T^2) definition the kernelized form must equal:
    o_t = sum_{i<=t} (q_t.k_i)^2 v_i / sum_{i<=t} (q_t.k_i)^2
    (KATA §1 and §2.2: normalised linear attention with the squared-inner-
    product kernel).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S = q @ k.T
    W = np.tril(S * S)
    num = W @ v
    den = W.sum(axis=1) + eps
    o = _safe_div(num, den)
    return (o, num, den) if return_parts else o


def prefill_bruteforce_rows(q, k, v, rows, eps: float = 0.0):
    """Brute-force outputs for selected rows only; O(t d) per row."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    out = np.zeros((len(rows), v.shape[1]))
    for r, t in enumerate(rows):
        w = (k[: t + 1] @ q[t]) ** 2
        den = w.sum() + eps
        out[r] = (w @ v[: t + 1]) / den if den != 0 else 0.0
    return out


def prefill_recurrent(q, k, v, H0=None, s0=None, eps: float = 0.0, return_parts: bool = False):
    """Token-by-token recurrence over the fixed-size state (H, s).

    KATA §1 (constant-time recurrent inference over a fixed-size state) and
    LoLA Metodologia item 2 (the state H_t and normaliser s_t). For each t:
    s += phi(k_t); H += phi(k_t) v_t^T; o_t = phi(q_t)^T H / (phi(q_t)^T s + eps).
    Returns o [T, dv], H [D, dv], s [D].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, d = q.shape
    dv = v.shape[1]
    D = phi_dim(d)
    H = np.zeros((D, dv)) if H0 is None else np.array(H0, np.float64, copy=True)
    s = np.zeros(D) if s0 is None else np.array(s0, np.float64, copy=True)
    o = np.zeros((T, dv))
    nums = np.zeros((T, dv))
    dens = np.zeros(T)
    for t in range(T):
        fk = phi(k[t])
        s += fk
        H += np.outer(fk, v[t])
        fq = phi(q[t])
        nums[t] = fq @ H
        dens[t] = fq @ s + eps
        o[t] = nums[t] / dens[t] if dens[t] != 0 else 0.0
    if return_parts:
        return o, H, s, nums, dens
    return o, H, s


def prefill_chunked(q, k, v, chunk: int = 256, H0=None, s0=None, eps: float = 0.0,
                    return_parts: bool = False):
    """Exact chunked form (KATA §2.3, "Paralelismo por Blocos" and the linear
    chunked-state operating point).

    Per chunk of rows Q, K, V:
      A   = lower-triangular part (with diagonal) of (Q K^T) o (Q K^T)
      num = A V + phi(Q) H          den = A 1 + phi(Q) s + eps
      o   = num / den
      then H += phi(K)^T V and s += phi(K)^T 1 carry the state to the next chunk.
    The cross-chunk carry is a running prefix sum of the chunk states, the
    sequential form of the page's associative scan.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, d = q.shape
    dv = v.shape[1]
    D = phi_dim(d)
    H = np.zeros((D, dv)) if H0 is None else np.array(H0, np.float64, copy=True)
    s = np.zeros(D) if s0 is None else np.array(s0, np.float64, copy=True)
    o = np.zeros((T, dv))
    nums = np.zeros((T, dv))
    dens = np.zeros(T)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        S = Q @ K.T
        A = np.tril(S * S)
        fQ = phi(Q)
        num = A @ V + fQ @ H
        den = A.sum(axis=1) + fQ @ s + eps
        nums[c0:c1] = num
        dens[c0:c1] = den
        o[c0:c1] = _safe_div(num, den)
        fK = phi(K)
        H += fK.T @ V
        s += fK.sum(axis=0)
    if return_parts:
        return o, H, s, nums, dens
    return o, H, s


def prefill(q, k, v, chunk: int = 256, H0=None, s0=None, eps: float = 0.0):
    """Batched chunked prefill: q, k [B, H, T, d], v [B, H, T, dv]; optional
    H0 [B, H, D, dv], s0 [B, H, D]. Returns o, H_T, s_T with leading [B, H]."""
    q = np.asarray(q)
    B, Hh, T, d = q.shape
    dv = np.shape(v)[-1]
    D = phi_dim(d)
    o = np.zeros((B, Hh, T, dv))
    HT = np.zeros((B, Hh, D, dv))
    sT = np.zeros((B, Hh, D))
    for b in range(B):
        for h in range(Hh):
            o[b, h], HT[b, h], sT[b, h] = prefill_chunked(
                q[b, h], k[b, h], v[b, h], chunk,
                None if H0 is None else H0[b, h], None if s0 is None else s0[b, h], eps)
    return o, HT, sT


# ----------------------------------------------------------------------------
# Backward: gradients of the causal prefill outputs
# ----------------------------------------------------------------------------

def prefill_backward(q, k, v, do, eps: float = 0.0):
    """Gradients of L = sum_t do_t . o_t with respect to q, k and v, for the
    causal prefill of KATA §1 with the lift of §2.2 written in its brute-force
    form (phi(q).phi(k) = (q.k)^2):
      s_ti = q_t . k_i,  w_ti = s_ti^2 (i <= t),  D_t = sum_i w_ti + eps,
      o_t = sum_i w_ti v_i / D_t  (0 when D_t is 0).
    The chain rule gives, with c_t = do_t . o_t,
      dv_i = sum_{t >= i} (w_ti / D_t) do_t,
      dw_ti = (do_t . v_i - c_t) / D_t,   ds_ti = 2 s_ti dw_ti,
      dq_t = sum_{i <= t} ds_ti k_i,      dk_i = sum_{t >= i} ds_ti q_t.
    Rows with D_t = 0 have a constant zero output and pass no gradient.
    Returns dq [T, d], dk [T, d], dv [T, dv] (float64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    S = np.tril(q @ k.T)
    W = S * S
    D = W.sum(axis=1) + eps
    live = D != 0
    inv = np.zeros_like(D)
    inv[live] = 1.0 / D[live]
    o = (W @ v) * inv[:, None]
    c = np.sum(do * o, axis=1)
    dv = (W * inv[:, None]).T @ do
    dW = ((do @ v.T) - c[:, None]) * inv[:, None]
    dS = np.tril(2.0 * S * dW)
    dq = dS @ k
    dk = dS.T @ q
    return dq, dk, dv


def prefill_backward_rows(q, k, v, do, q_rows, k_rows, eps: float = 0.0, chunk: int = 256):
    """prefill_backward for selected rows only: dq at the queries q_rows and
    dk, dv at the keys k_rows, each in O(T (d + d_v)) once every o_t and D_t
    are known (from the chunked form). Same formulas as prefill_backward."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    o, _, _, _, D = prefill_chunked(q, k, v, chunk=chunk, eps=eps, return_parts=True)
    live = D != 0
    inv = np.zeros_like(D)
    inv[live] = 1.0 / D[live]
    c = np.sum(do * o, axis=1)
    dq = np.zeros((len(q_rows), q.shape[1]))
    for r, t in enumerate(q_rows):
        st = k[: t + 1] @ q[t]
        dw = (v[: t + 1] @ do[t] - c[t]) * inv[t]
        dq[r] = (2.0 * st * dw) @ k[: t + 1]
    dk = np.zeros((len(k_rows), k.shape[1]))
    dv = np.zeros((len(k_rows), v.shape[1]))
    for r, i in enumerate(k_rows):
        si = q[i:] @ k[i]
        dv[r] = (si * si * inv[i:]) @ do[i:]
        dw = (do[i:] @ v[i] - c[i:]) * inv[i:]
        dk[r] = (2.0 * si * dw) @ q[i:]
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Decode step, self-recall error, selection
# ----------------------------------------------------------------------------

def decode_step(H, s, q, k, v, eps: float = 0.0):
    """One recurrent token: the state absorbs (k, v) first, then q reads it
    out, since H_t sums over i <= t (KATA §1; LoLA Estratégia de Inferência,
    token-by-token mode). Returns o [dv], H' [D, dv], s' [D]."""
    fk = phi(k)
    s2 = np.asarray(s, np.float64) + fk
    H2 = np.asarray(H, np.float64) + np.outer(fk, np.asarray(v, np.float64))
    fq = phi(q)
    den = fq @ s2 + eps
    o = (fq @ H2) / den if den != 0 else np.zeros(H2.shape[1])
    return o, H2, s2


def sre(H, s, k, v, eps: float = 0.0):
    """Self-recall error of LoLA ("O Mecanismo de Erro de Auto-Recuperação"):
    SRE(k, v | H, s) = || phi(k)^T H / phi(k)^T s - v ||^2, for a batch of
    candidate pairs k [n, d], v [n, dv]. A zero denominator predicts 0."""
    fk = phi(np.asarray(k, np.float64))
    num = fk @ np.asarray(H, np.float64)
    den = fk @ np.asarray(s, np.float64) + eps
    pred = _safe_div(num, den)
    r = pred - np.asarray(v, np.float64)
    return np.sum(r * r, axis=-1)


def sre_bruteforce(keys, values, k, v):
    """Self-recall error against the state made of the pairs (keys_i, values_i),
    without forming the state: pred = sum_i (k.k_i)^2 v_i / sum_i (k.k_i)^2."""
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    k = np.atleast_2d(np.asarray(k, np.float64))
    v = np.atleast_2d(np.asarray(v, np.float64))
    out = np.zeros(k.shape[0])
    for c in range(k.shape[0]):
        w = (keys @ k[c]) ** 2 if len(keys) else np.zeros(0)
        den = w.sum()
        pred = (w @ values) / den if den != 0 else np.zeros(v.shape[1])
        out[c] = np.sum((pred - v[c]) ** 2)
    return out


def select_topk(scores, m: int, ids=None) -> np.ndarray:
    """Positions of the m highest scores, ordered by (score descending, id
    ascending); ``ids`` defaults to the positions themselves. LoLA
    Estratégia de Inferência, item 2: the highest-SRE pairs are kept."""
    scores = np.asarray(scores, np.float64)
    ids = np.arange(len(scores)) if ids is None else np.asarray(ids)
    order = np.lexsort((ids, -scores))
    return order[:m]


def near_tie_ok(oracle_scores, chosen, m: int, rel: float = 1e-5) -> bool:
    """Whether the set ``chosen`` (positions) is an acceptable top-m of
    ``oracle_scores``: equal to the oracle's set when the boundary gap is
    wider than ``rel``; otherwise every chosen score reaches s_(m)(1-rel)
    and every score above s_(m)(1+rel) is chosen."""
    sc = np.asarray(oracle_scores, np.float64)
    chosen = np.asarray(chosen)
    if len(set(chosen.tolist())) != len(chosen) or len(chosen) != min(m, len(sc)):
        return False
    if m <= 0:
        return len(chosen) == 0
    if m >= len(sc):
        return set(chosen.tolist()) == set(range(len(sc)))
    srt = np.sort(sc)[::-1]
    sm, sm1 = srt[m - 1], srt[m]
    gap = (sm - sm1) / sm if sm != 0 else (0.0 if sm1 == sm else np.inf)
    ref = set(select_topk(sc, m).tolist())
    if gap > rel:
        return set(chosen.tolist()) == ref
    lo = sm * (1 - rel)
    hi = sm * (1 + rel)
    if np.any(sc[chosen] < lo):
        return False
    must = set(np.nonzero(sc > hi)[0].tolist())
    return must.issubset(set(chosen.tolist()))


# ----------------------------------------------------------------------------
# Decode + sparse-cache selection chain
# ----------------------------------------------------------------------------

def decode_sre_chain(H0, s0, q, k, v, fresh_k, fresh_v, cache_k, cache_v, top_k: int,
                     eps: float = 0.0, choose: Optional[Callable] = None):
    """One head-state through S decode steps with self-recall selection.

    Per step tau: (i) decode_step with (q, k, v)[tau]; (ii) candidates are the
    current cache pairs (slot order) followed by the fresh pairs of this step;
    (iii) every candidate is scored by SRE against the updated state;
    (iv) the top_k candidates by (score desc, slot asc) become the next cache
    in that order; (v) the rest are discarded.

    q, k, v: [S, d]; fresh_k, fresh_v: [S, n_fresh, d]; cache_k, cache_v:
    [top_k, d]. ``choose(tau, scores, sel)`` may return a replacement
    selection (used to follow the GPU through near-ties).
    Returns dict with o [S, dv], scores [S, n_cand], sel [S, top_k], H, s,
    cache_k, cache_v.
    """
    H = np.array(H0, np.float64, copy=True)
    s = np.array(s0, np.float64, copy=True)
    ck = np.asarray(cache_k, np.float64)
    cv = np.asarray(cache_v, np.float64)
    S = len(q)
    outs, scs, sels = [], [], []
    for tau in range(S):
        o, H, s = decode_step(H, s, q[tau], k[tau], v[tau], eps)
        cand_k = np.concatenate([ck, np.asarray(fresh_k[tau], np.float64)], axis=0)
        cand_v = np.concatenate([cv, np.asarray(fresh_v[tau], np.float64)], axis=0)
        sc = sre(H, s, cand_k, cand_v, eps)
        sel = select_topk(sc, top_k)
        if choose is not None:
            sel = np.asarray(choose(tau, sc, sel))
        ck, cv = cand_k[sel], cand_v[sel]
        outs.append(o)
        scs.append(sc)
        sels.append(sel)
    return dict(o=np.array(outs), scores=np.array(scs), sel=np.array(sels), H=H, s=s,
                cache_k=ck, cache_v=cv)


# ----------------------------------------------------------------------------
# Hybrid: sliding window + linear state + sparse cache (one head)
# ----------------------------------------------------------------------------

def hybrid_prefill(q, k, v, window: int, cache_size: int, refresh: int, scale: float,
                   eps: float = 0.0, choose: Optional[Callable] = None):
    """LoLA's three memories over one head, processed in blocks of ``refresh``
    tokens (LoLA Metodologia items 1-3 and Estratégia de Inferência items 1-4).

    For block b covering tokens [bR, min(T, bR+R)):
      1. eviction frontier f = max(0, bR - window); the tokens [f_prev, f)
         leave the window;
      2. candidates = cache + evicted. If there are at most cache_size of
         them they all stay in the cache. Otherwise each candidate is scored
         by SRE against the current (H, s) (before this refresh's fold), the
         cache_size highest (score desc, token id asc) stay, and every other
         candidate is folded into the state: H += phi(k_i) v_i^T,
         s += phi(k_i);
      3. each query t of the block reads one jointly normalised mixture:
         num = sum_{i in [f, t]} e^{scale q_t.k_i} v_i
             + sum_{j in cache} e^{scale q_t.k_j} v_j + phi(q_t)^T H
         den = the same sums without v, plus phi(q_t)^T s, plus eps;
         o_t = num / den.
    ``choose(block, cand_ids, scores, keep_ids)`` may replace the kept set.
    Returns dict: o [T, dv], H, s, cache (sorted token ids), trace {block:
    sorted kept ids}, refreshes (number of scored refreshes).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, d = q.shape
    dv = v.shape[1]
    D = phi_dim(d)
    H = np.zeros((D, dv))
    s = np.zeros(D)
    cache: list = []
    f_prev = 0
    o = np.zeros((T, dv))
    trace = {}
    nref = 0
    nblocks = -(-T // refresh)
    for b in range(nblocks):
        b0, b1 = b * refresh, min(T, (b + 1) * refresh)
        f = max(0, b0 - window)
        evicted = list(range(f_prev, f))
        f_prev = f
        if evicted:
            cand = cache + evicted
            if len(cand) <= cache_size:
                cache = cand
            else:
                ids = np.array(cand)
                sc = sre(H, s, k[ids], v[ids], eps)
                pos = select_topk(sc, cache_size, ids=ids)
                keep = ids[pos]
                if choose is not None:
                    keep = np.asarray(choose(b, ids, sc, keep))
                keep_set = set(int(x) for x in keep)
                rejected = [int(i) for i in ids if int(i) not in keep_set]
                if rejected:
                    fK = phi(k[rejected])
                    H += fK.T @ v[rejected]
                    s += fK.sum(axis=0)
                cache = sorted(keep_set)
                trace[b] = sorted(keep_set)
                nref += 1
        cidx = np.array(cache, dtype=int)
        fQ = phi(q[b0:b1])
        for t in range(b0, b1):
            w_win = np.exp(scale * (k[f:t + 1] @ q[t]))
            num = w_win @ v[f:t + 1]
            den = w_win.sum()
            if len(cidx):
                w_c = np.exp(scale * (k[cidx] @ q[t]))
                num = num + w_c @ v[cidx]
                den = den + w_c.sum()
            fq = fQ[t - b0]
            num = num + fq @ H
            den = den + fq @ s + eps
            o[t] = num / den if den != 0 else 0.0
    return dict(o=o, H=H, s=s, cache=sorted(cache), trace=trace, refreshes=nref)
