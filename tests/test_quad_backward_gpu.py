"""GPU parity of the prefill gradients (kla_prefill_quadratic_backward)
against the float64 oracle (oracle.prefill_backward, pinned on the CPU by
finite differences and homogeneity identities).

The forward runs on the GPU (kla_prefill_quadratic with its row
denominators); the oracle recomputes everything in float64 from the same
bf16 inputs and output gradients. Every row is compared at sizes the oracle finishes in seconds,
sampled rows at the full prefill_4x8x4096 size. Tolerance: the bf16 bound.
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


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _case(B, H, T, seed, dtype):
    c = S.prefill_case("bwd", B, H, T, 64, 64, 64, seed=seed)
    rng = np.random.default_rng(seed + 1)
    g = S.round_to_bf16(S.gaussian(rng, (B, H, T, 64)))
    q, k, v = (dev(x, torch.bfloat16) for x in (c.q, c.k, c.v))
    return c, g, q, k, v, dev(g, dtype)


def _gpu_grads(K, q, k, v, g, eps, out_dtype):
    o, den = K.prefill_quadratic(q, k, v, eps=eps, out_dtype=out_dtype, return_den=True)
    dq, dk, dv = K.prefill_quadratic_backward(q, k, v, den, g.to(out_dtype), eps=eps)
    torch.cuda.synchronize()
    return o, den, dq, dk, dv


def _close_or_zero(x, r, scale, what):
    # a gradient that is exactly zero in exact arithmetic (a lone token's
    # query and key) is compared in absolute terms against the data's scale
    if float(np.sqrt(np.mean(r * r))) < 1e-9 * scale:
        assert float(np.abs(x).max()) <= 1e-4 * scale, f"{what}: {np.abs(x).max()} not ~0"
    else:
        assert_close(x, r, RTOL_BF16, what)


@pytest.mark.parametrize("T", [1, 5, 64, 100, 129, 300])
@pytest.mark.parametrize("out_dtype,eps", [(torch.bfloat16, 0.0), (torch.float32, 0.0), (torch.float32, 0.25)])
def test_backward_every_row(K, T, out_dtype, eps):
    # the exact gradients of the float64 oracle, in bf16 or float32
    B, H = 1, 2
    c, g, q, k, v, gd = _case(B, H, T, 600 + T, out_dtype)
    o, den, dq, dk, dv = _gpu_grads(K, q, k, v, gd, eps, out_dtype)
    assert dq.dtype == out_dtype and dq.shape == (B, H, T, 64)
    for h in range(H):
        _, _, ref_den = O.prefill_bruteforce(c.q[0, h], c.k[0, h], c.v[0, h], eps=eps, return_parts=True)
        assert_close(host(den)[0, h], ref_den, RTOL_BF16, f"den head {h} T={T}")
        rq, rk, rv = O.prefill_backward(c.q[0, h], c.k[0, h], c.v[0, h], g[0, h], eps=eps)
        scale = float(np.abs(g[0, h]).max())
        _close_or_zero(host(dq)[0, h], rq, scale, f"dq head {h} T={T}")
        _close_or_zero(host(dk)[0, h], rk, scale, f"dk head {h} T={T}")
        assert_close(host(dv)[0, h], rv, RTOL_BF16, f"dv head {h} T={T}")


def test_backward_degenerate(K):
    # zero queries pass no gradient to q or k (D = 0) and none to v; a single
    # token's value gradient is its output gradient
    T = 130
    z = torch.zeros((1, 1, T, 64), device="cuda", dtype=torch.bfloat16)
    kk = torch.randn((1, 1, T, 64), device="cuda").to(torch.bfloat16)
    vv = torch.randn((1, 1, T, 64), device="cuda").to(torch.bfloat16)
    gg = torch.randn((1, 1, T, 64), device="cuda").to(torch.bfloat16)
    _, _, dq, dk, dv = _gpu_grads(K, z, kk, vv, gg, 0.0, torch.bfloat16)
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)
    q1, k1, v1 = (torch.randn((2, 3, 1, 64), device="cuda").to(torch.bfloat16) for _ in range(3))
    g1 = torch.randn((2, 3, 1, 64), device="cuda")
    _, _, dq, dk, dv = _gpu_grads(K, q1, k1, v1, g1, 0.0, torch.float32)
    assert_close(host(dv), host(g1), RTOL_BF16, "T=1 dv")
    assert float(dq.abs().max()) < 1e-3 * float(g1.float().abs().max()) + 1e-6
    assert float(dk.abs().max()) < 1e-3 * float(g1.float().abs().max()) + 1e-6


def test_backward_4x8x4096_full_size(K):
    # the headline prefill workload: sampled rows of every gradient for two
    # heads against the oracle's row form (float32 outputs)
    cfg = S.CONFIGS["prefill_4x8x4096"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    c = S.prefill_case("prefill_4x8x4096", B, H, T, cfg["d_qk"], cfg["d_v"], cfg["chunk"], cfg["seed"])
    rng = np.random.default_rng(77)
    g = S.round_to_bf16(S.gaussian(rng, (B, H, T, 64)))
    q, k, v = (dev(x, torch.bfloat16) for x in (c.q, c.k, c.v))
    _, _, dq, dk, dv = _gpu_grads(K, q, k, v, dev(g), 0.0, torch.float32)
    gq, gk, gv = host(dq), host(dk), host(dv)
    for (b, h) in [(0, 0), (B - 1, H - 1)]:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, T - 1], rng.integers(0, T, 12)]))
        rq, rk, rv = O.prefill_backward_rows(c.q[b, h], c.k[b, h], c.v[b, h], g[b, h], rows, rows)
        assert_close(gq[b, h, rows], rq, RTOL_BF16, f"dq rows head ({b},{h})")
        assert_close(gk[b, h, rows], rk, RTOL_BF16, f"dk rows head ({b},{h})")
        assert_close(gv[b, h, rows], rv, RTOL_BF16, f"dv rows head ({b},{h})")
