"""Seeded synthetic inputs for causal kernelized linear attention.

This module only draws and shapes random numbers. It holds none of the
method's arithmetic: no feature lift, no attention, no state, no scoring.
Both the GPU path (through the tests and the benchmark) and the float64 CPU
oracle consume what it returns, so the two sides always see bit-identical
inputs.

Generator: ``numpy.random.default_rng([seed, *stream_ids])`` (PCG64), one
stream per attention head (or per decode head-state), so that any subset of
heads can be regenerated on the host on its own.

Workload shapes follow the pages' workloads:
  * KATA page ("Kernelized Linear Attention: Breaking the Capacity Wall with
    Symmetric Cones"), §2.3 and §4: long-sequence throughput of the exact
    chunked-state form (the 131k-token kernel run stands behind the
    long-context prefill below);
  * LoLA page ("LoLA: Atenção Linear de Baixo Rank com Cache Esparso"),
    Metodologia and Estratégia de Inferência: a sliding window, a linear
    state and a sparse cache refreshed by self-recall error; the recall
    suites the pages evaluate on are not reproduced; keys with injected
    near-duplicates stand in for their colliding keys.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "round_to_bf16",
    "gaussian",
    "l2_normalised",
    "PrefillCase",
    "prefill_case",
    "DecodeCase",
    "decode_case",
    "HybridCase",
    "hybrid_case",
    "hybrid_head",
    "hybrid_decode_tokens",
    "DecodeStream",
    "CONFIGS",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16, so a
    later ``torch.bfloat16`` conversion is exact and the float64 view used by
    the oracle holds the very same numbers.
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def gaussian(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """float32 standard normal draws times ``scale`` (a power of two keeps it exact)."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    return z


def l2_normalised(z: np.ndarray) -> np.ndarray:
    """Rows divided by their Euclidean norm, in float32."""
    n = np.sqrt(np.sum(z.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    n[n == 0] = 1
    return (z / n).astype(np.float32)


# ----------------------------------------------------------------------------
# Prefill workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillCase:
    """q, k: [B, H, T, d_qk]; v: [B, H, T, d_v]; float32 arrays holding the
    exact values the GPU receives (already bf16-rounded when ``dtype`` is
    ``"bf16"``)."""

    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    chunk: int
    dtype: str  # "f32" or "bf16"
    heads: tuple = ()  # (b, h) pairs that were generated, in order


def _prefill_head(seed, b, h, T, d_qk, d_v, kind):
    rng = np.random.default_rng([seed, b, h])
    if kind == "tiny":
        s = 1.0 / math.sqrt(d_qk)
        q = gaussian(rng, (T, d_qk), s)
        k = gaussian(rng, (T, d_qk), s)
        v = gaussian(rng, (T, d_v), s)
        return q, k, v
    q = round_to_bf16(l2_normalised(gaussian(rng, (T, d_qk))))
    k = round_to_bf16(l2_normalised(gaussian(rng, (T, d_qk))))
    v = round_to_bf16(gaussian(rng, (T, d_v)))
    return q, k, v


def prefill_case(name: str, B: int, H: int, T: int, d_qk: int, d_v: int, chunk: int,
                 seed: int, kind: str = "normalised", heads=None, threads: int = 8) -> PrefillCase:
    """Generate a prefill workload.

    kind = "tiny": q, k, v i.i.d. N(0,1)/sqrt(d_qk), float32.
    kind = "normalised": q, k rows are L2-normalised N(0, I) draws and
    v ~ N(0,1), all rounded to bf16.

    ``heads`` restricts generation to a list of (b, h) pairs; the arrays then
    have shape [1, len(heads), T, d] in that order.
    """
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
        shape_bh = (B, H)
    else:
        heads = [tuple(x) for x in heads]
        shape_bh = (1, len(heads))
    n = len(heads)
    q = np.empty((n, T, d_qk), np.float32)
    k = np.empty((n, T, d_qk), np.float32)
    v = np.empty((n, T, d_v), np.float32)

    def work(i):
        b, h = heads[i]
        q[i], k[i], v[i] = _prefill_head(seed, b, h, T, d_qk, d_v, kind)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, range(n)))
    dtype = "f32" if kind == "tiny" else "bf16"
    return PrefillCase(name, q.reshape(*shape_bh, T, d_qk), k.reshape(*shape_bh, T, d_qk),
                       v.reshape(*shape_bh, T, d_v), chunk, dtype, tuple(heads))


# ----------------------------------------------------------------------------
# Decode + self-recall-error selection workload
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeCase:
    """Per head-state n (N of them):
      prefix_k, prefix_v: [N, T0, d] build the initial state (q is not needed
        for the state, so the prefix queries are the prefix keys);
      cache0_k, cache0_v: [N, top_k, d] initial sparse-cache contents;
      q, k, v: [S, N, d] the token of each step;
      fresh_k, fresh_v: [S, N, n_fresh, d] fresh candidate pairs of each step.
    All float32. Keys and queries are N(0,1)/sqrt(d); values N(0,1).
    """

    N: int
    d: int
    steps: int
    top_k: int
    n_fresh: int
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    cache0_k: np.ndarray
    cache0_v: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    fresh_k: np.ndarray
    fresh_v: np.ndarray
    ids: tuple = ()


def decode_case(N: int, d: int = 64, T0: int = 2048, steps: int = 128, top_k: int = 16,
                n_fresh: int = 48, seed: int = 4, ids=None, threads: int = 8) -> DecodeCase:
    """Generate the decode workload for head-states ``ids`` (default 0..N-1).

    Draw order per head-state n, from default_rng([seed, n]): prefix k, prefix
    v, cache0 k, cache0 v, then one row per step holding q, k, v, fresh k and
    fresh v, so a run of S steps is a prefix of any longer run.
    """
    ids = tuple(range(N)) if ids is None else tuple(int(i) for i in ids)
    n = len(ids)
    s = 1.0 / math.sqrt(d)
    pk = np.empty((n, T0, d), np.float32)
    pv = np.empty((n, T0, d), np.float32)
    ck = np.empty((n, top_k, d), np.float32)
    cv = np.empty((n, top_k, d), np.float32)
    q = np.empty((steps, n, d), np.float32)
    k = np.empty((steps, n, d), np.float32)
    v = np.empty((steps, n, d), np.float32)
    fk = np.empty((steps, n, n_fresh, d), np.float32)
    fv = np.empty((steps, n, n_fresh, d), np.float32)

    def work(i):
        rng = np.random.default_rng([seed, ids[i]])
        pk[i] = gaussian(rng, (T0, d), s)
        pv[i] = gaussian(rng, (T0, d))
        ck[i] = gaussian(rng, (top_k, d), s)
        cv[i] = gaussian(rng, (top_k, d))
        # one row per step: [q | k | v | fresh k | fresh v]; the stream is
        # sequential, so the first S rows do not depend on ``steps``
        rows = gaussian(rng, (steps, (3 + 2 * n_fresh) * d))
        sc = np.float32(s)
        q[:, i] = rows[:, 0:d] * sc
        k[:, i] = rows[:, d:2 * d] * sc
        v[:, i] = rows[:, 2 * d:3 * d]
        fk[:, i] = rows[:, 3 * d:(3 + n_fresh) * d].reshape(steps, n_fresh, d) * sc
        fv[:, i] = rows[:, (3 + n_fresh) * d:].reshape(steps, n_fresh, d)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, range(n)))
    return DecodeCase(n, d, steps, top_k, n_fresh, pk, pv, ck, cv, q, k, v, fk, fv, ids)


class DecodeStream:
    """The draws of ``decode_case``, one step at a time.

    Construction draws every head-state's prefix and initial cache (the
    ``prefix_k``, ``prefix_v``, ``cache0_k``, ``cache0_v`` attributes, as in
    DecodeCase); each ``next_step()`` then draws the following step's row of
    q, k, v and fresh candidates for every head-state, from the same
    per-head-state generators and in the same order, so the values equal
    ``decode_case(...)`` for the same arguments while only one step is held
    in memory (the full workload's 128 steps of fresh candidates take 13 GB).
    Returns (q, k, v, fresh_k, fresh_v) shaped [N, d], [N, n_fresh, d].
    """

    def __init__(self, N: int, d: int = 64, T0: int = 2048, top_k: int = 16, n_fresh: int = 48,
                 seed: int = 4, ids=None, threads: int = 8):
        self.ids = tuple(range(N)) if ids is None else tuple(int(i) for i in ids)
        n = len(self.ids)
        self.N, self.d, self.top_k, self.n_fresh, self.threads = n, d, top_k, n_fresh, threads
        self.scale = np.float32(1.0 / math.sqrt(d))
        self.rngs = [np.random.default_rng([seed, i]) for i in self.ids]
        s = 1.0 / math.sqrt(d)
        self.prefix_k = np.empty((n, T0, d), np.float32)
        self.prefix_v = np.empty((n, T0, d), np.float32)
        self.cache0_k = np.empty((n, top_k, d), np.float32)
        self.cache0_v = np.empty((n, top_k, d), np.float32)

        def work(i):
            rng = self.rngs[i]
            self.prefix_k[i] = gaussian(rng, (T0, d), s)
            self.prefix_v[i] = gaussian(rng, (T0, d))
            self.cache0_k[i] = gaussian(rng, (top_k, d), s)
            self.cache0_v[i] = gaussian(rng, (top_k, d))

        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(work, range(n)))

    def drop_prefix(self):
        """Release the prefix arrays once the initial state is built."""
        self.prefix_k = self.prefix_v = None

    def next_step(self):
        n, d, nf, sc = self.N, self.d, self.n_fresh, self.scale
        rows = np.empty((n, (3 + 2 * nf) * d), np.float32)

        def work(i):
            rows[i] = gaussian(self.rngs[i], (1, (3 + 2 * nf) * d))[0]

        with ThreadPoolExecutor(max_workers=max(1, self.threads)) as ex:
            list(ex.map(work, range(n)))
        q = rows[:, 0:d] * sc
        k = rows[:, d:2 * d] * sc
        v = rows[:, 2 * d:3 * d].copy()
        fk = rows[:, 3 * d:(3 + nf) * d].reshape(n, nf, d) * sc
        fv = rows[:, (3 + nf) * d:].reshape(n, nf, d).copy()
        return q, k, v, fk, fv


# ----------------------------------------------------------------------------
# Hybrid (window + linear state + sparse cache) workload
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class HybridCase:
    name: str
    q: np.ndarray  # [B, H, T, d] bf16-exact float32
    k: np.ndarray
    v: np.ndarray
    window: int
    cache_size: int
    refresh: int
    dup_positions: tuple = ()  # per head: positions turned into near-duplicates


def _hybrid_head(seed, b, h, T, d, dup_frac, noise, min_cos):
    rng = np.random.default_rng([seed, b, h])
    q = round_to_bf16(l2_normalised(gaussian(rng, (T, d))))
    k = round_to_bf16(l2_normalised(gaussian(rng, (T, d))))
    v = round_to_bf16(gaussian(rng, (T, d)))
    m = int(round(dup_frac * T))
    m = min(m, max(T - 1, 0))
    pos = np.sort(rng.choice(np.arange(1, T), size=m, replace=False)) if m > 0 else np.zeros(0, int)
    for t in pos:
        src = int(rng.integers(0, t))
        base = k[src].astype(np.float32)
        while True:
            z = gaussian(rng, (d,))
            cand = round_to_bf16(l2_normalised((base + np.float32(noise) * z)[None, :]))[0]
            c = float(np.dot(cand.astype(np.float64), base.astype(np.float64))
                      / (np.linalg.norm(cand.astype(np.float64)) * np.linalg.norm(base.astype(np.float64))))
            if c > min_cos:
                k[t] = cand
                break
    return q, k, v, tuple(int(p) for p in pos)


def hybrid_head(seed: int, b: int, h: int, T: int, d: int, dup_frac: float = 0.05, noise: float = 0.04,
                min_cos: float = 0.9):
    """Head (b, h) of hybrid_case on its own: (q, k, v, near-duplicate positions)."""
    return _hybrid_head(seed, b, h, T, d, dup_frac, noise, min_cos)


def hybrid_case(name: str, B: int, H: int, T: int, d: int, window: int, cache_size: int,
                refresh: int, seed: int, dup_frac: float = 0.05, noise: float = 0.04,
                min_cos: float = 0.9, threads: int = 8) -> HybridCase:
    """q, k rows L2-normalised Gaussian, v ~ N(0,1), all bf16-rounded; then a
    fraction ``dup_frac`` of key positions t (drawn without replacement from
    [1, T)) is replaced, in increasing t, by a noisy copy of an earlier key
    k_src (src ~ U[0, t)) with cosine above ``min_cos`` after rounding."""
    q = np.empty((B * H, T, d), np.float32)
    k = np.empty((B * H, T, d), np.float32)
    v = np.empty((B * H, T, d), np.float32)
    dups = [None] * (B * H)

    def work(i):
        b, h = divmod(i, H)
        q[i], k[i], v[i], dups[i] = _hybrid_head(seed, b, h, T, d, dup_frac, noise, min_cos)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, range(B * H)))
    return HybridCase(name, q.reshape(B, H, T, d), k.reshape(B, H, T, d), v.reshape(B, H, T, d),
                      window, cache_size, refresh, tuple(dups))


def hybrid_decode_tokens(N: int, T: int, d: int, seed: int, dup_frac: float = 0.05,
                         noise: float = 0.04, device="cuda"):
    """Token stream of the token-by-token hybrid decode, drawn on ``device``
    with torch's seeded generator (too large to draw per head on the host):
    q, k, v as [T, N, d] bfloat16. q, k rows are L2-normalised Gaussian and
    v ~ N(0,1), as in hybrid_case. Each key position t >= 1 independently
    becomes, with probability ``dup_frac``, a near-duplicate
    normalise(k0_src + noise * z) of an earlier original key k0_src,
    src ~ U[0, t) (no cosine re-draw: with noise 0.04 in d = 64 the cosine
    is about 0.95). The tests copy sampled heads back to the host, so the
    oracle sees the same values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))

    def unit_rows():
        x = torch.randn((T, N, d), generator=g, device=device, dtype=torch.float32)
        return x / x.norm(dim=-1, keepdim=True)

    q = unit_rows().to(torch.bfloat16)
    k0 = unit_rows()
    v = torch.randn((T, N, d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    dup = torch.rand((T, N), generator=g, device=device) < dup_frac
    dup[0] = False
    tt, nn = dup.nonzero(as_tuple=True)
    src = (torch.rand(tt.shape, generator=g, device=device) * tt.to(torch.float32)).long()
    src = torch.minimum(src, tt - 1)
    z = torch.randn((tt.numel(), d), generator=g, device=device, dtype=torch.float32)
    kd = k0[src, nn] + float(noise) * z
    k = k0.clone()
    k[tt, nn] = kd / kd.norm(dim=-1, keepdim=True)
    del k0
    return q, k.to(torch.bfloat16), v


# ----------------------------------------------------------------------------
# The workloads
# ----------------------------------------------------------------------------

CONFIGS = {
    # tiny fp32 causal case, parity only
    "tiny_f32": dict(kind="prefill", B=1, H=1, T=256, d_qk=16, d_v=16, chunk=32, seed=1,
                     gen="tiny"),
    # bf16 prefill, 4 x 8 heads x 4096 tokens, d = 64, chunk 64
    "prefill_4x8x4096": dict(kind="prefill", B=4, H=8, T=4096, d_qk=64, d_v=64, chunk=64,
                             seed=2, gen="normalised"),
    # long-context bf16 prefill, 16 heads x 65536 tokens, chunk 128
    "prefill_1x16x65536": dict(kind="prefill", B=1, H=16, T=65536, d_qk=64, d_v=64,
                               chunk=128, seed=3, gen="normalised"),
    # recurrent decode + SRE top-16 of 64 candidates, 256 seq x 16 heads, 128 steps
    "decode_sre_4096x128": dict(kind="decode", N=4096, d=64, T0=2048, steps=128, top_k=16,
                                n_fresh=48, seed=4),
    # hybrid prefill: window 512, sparse cache 128, refresh every 64 tokens
    "hybrid_2x16x16384": dict(kind="hybrid", B=2, H=16, T=16384, d=64, window=512,
                              cache_size=128, refresh=64, seed=5),
    # token-by-token hybrid decode with the hybrid prefill's memories (window
    # 512, cache 128) over the decode workload's 256 seq x 16 heads: 2048
    # tokens bring every head-state to a full window and cache, then 128 steps
    "hybrid_decode_4096": dict(kind="hybrid_decode", N=4096, d=64, window=512, cache_size=128,
                               T0=2048, steps=128, seed=6, dup_frac=0.05),
}
