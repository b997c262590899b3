"""GPU parity of the multi-factor variants in the quadratic form
(kla_prefill_quadratic_factors: KATA-Mg "concat" and KATA-Sigma-g "sum")
against the float64 oracle (oracle.prefill_factors_bruteforce, pinned on the
CPU by a hand-worked example, closed forms, symmetries and its state form).
Every row at small sizes, sampled rows at the full prefill_4x8x4096 size.
Tolerance: the bf16 bound.
"""
import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_02_amd import synth as S
from tests.tolerance import RTOL_BF16, assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kernelized_linear_attention_02_amd as K
    K.load_library()
    return K


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kind", ["concat", "sum"])
@pytest.mark.parametrize("g", [1, 2, 4])
@pytest.mark.parametrize("T,out_dtype,eps", [(1, torch.bfloat16, 0.0), (100, torch.float32, 0.0),
                                             (300, torch.bfloat16, 0.0), (257, torch.float32, 0.3)])
def test_factors_every_row(K, kind, g, T, out_dtype, eps):
    B, H = 1, 2
    c = S.prefill_case("factors", B, H, T, 64, 64, 64, seed=900 + T + 10 * g)
    o, den = K.prefill_quadratic(dev(c.q), dev(c.k), dev(c.v), eps=eps, out_dtype=out_dtype, return_den=True,
                                 factors=g, factor_kind=kind)
    torch.cuda.synchronize()
    assert o.dtype == out_dtype
    for h in range(H):
        ro, _, rden = O.prefill_factors_bruteforce(c.q[0, h], c.k[0, h], c.v[0, h], g, kind, eps=eps,
                                                   return_parts=True)
        assert_close(host(o)[0, h], ro, RTOL_BF16, f"o {kind} g={g} head {h}")
        assert_close(host(den)[0, h], rden, RTOL_BF16, f"den {kind} g={g} head {h}")


def test_factors_one_is_the_rank_one_form(K):
    # factors = 1 runs the same arithmetic as kla_prefill_quadratic, either kind
    c = S.prefill_case("factors1", 1, 3, 200, 64, 64, 64, seed=42)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    base = K.prefill_quadratic(q, k, v, out_dtype=torch.float32)
    for kind in ("concat", "sum"):
        o = K.prefill_quadratic(q, k, v, out_dtype=torch.float32, factors=1, factor_kind=kind)
        assert torch.equal(o, base)


def test_factors_differ_from_rank_one(K):
    # the variants compute different functions (guards against a silent fallback)
    c = S.prefill_case("factors2", 1, 1, 128, 64, 64, 64, seed=43)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    outs = [host(K.prefill_quadratic(q, k, v, out_dtype=torch.float32, factors=g, factor_kind=kind))
            for g, kind in [(1, "concat"), (2, "concat"), (2, "sum"), (4, "concat"), (4, "sum")]]
    for a in range(len(outs)):
        for b in range(a + 1, len(outs)):
            assert np.max(np.abs(outs[a] - outs[b])) > 1e-3


@pytest.mark.parametrize("kind", ["concat", "sum"])
def test_factors_4x8x4096_full_size(K, kind):
    cfg = S.CONFIGS["prefill_4x8x4096"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    c = S.prefill_case("prefill_4x8x4096", B, H, T, cfg["d_qk"], cfg["d_v"], cfg["chunk"], cfg["seed"])
    o = K.prefill_quadratic(dev(c.q), dev(c.k), dev(c.v), out_dtype=torch.float32, factors=2, factor_kind=kind)
    go = host(o)
    rng = np.random.default_rng(5)
    for (b, h) in [(0, 0), (B - 1, H - 1)]:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, T - 1], rng.integers(0, T, 12)]))
        # the oracle's closed-form weights for the sampled query rows, causal
        W = np.where(np.arange(T)[None, :] <= rows[:, None], O.factor_weights(c.q[b, h][rows], c.k[b, h], 2, kind), 0.0)
        ref = (W @ c.v[b, h].astype(np.float64)) / W.sum(axis=1)[:, None]
        assert_close(go[b, h, rows], ref, RTOL_BF16, f"o rows {kind} head ({b},{h})")
