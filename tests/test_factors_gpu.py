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
from tests.tolerance import RTOL_BF16, RTOL_F32, assert_close

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


# ---- the concatenated lift through the chunked state form (kla_prefill_factors)

@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("B,H,chunk,T", [(1, 3, 64, 50), (2, 2, 128, 300), (2, 10, 64, 130), (1, 17, 32, 97)])
def test_factors_state_form_every_row(K, g, B, H, chunk, T):
    # against the oracle's fixed-size state form: outputs and the final state
    # (H_T, s_T in the concatenated per-factor vec_sym layout); more than 16
    # heads exercises the 8-slice split
    c = S.prefill_case("factors_state", B, H, T, 64, 64, chunk, seed=70 + g + T)
    o, HT, sT = K.prefill(dev(c.q), dev(c.k), dev(c.v), chunk=chunk, return_state=True, factors=g)
    torch.cuda.synchronize()
    D = K.factor_phi_dim(64, g)
    assert HT.shape == (B, H, D, 64) and sT.shape == (B, H, D)
    for b in range(B):
        for h in range(H):
            ro, rH, rs = O.prefill_factors_recurrent(c.q[b, h], c.k[b, h], c.v[b, h], g, "concat")
            assert_close(host(o)[b, h], ro, RTOL_BF16, f"o g={g} head ({b},{h})")
            assert_close(host(HT)[b, h], rH, RTOL_BF16, f"H_T g={g} head ({b},{h})")
            assert_close(host(sT)[b, h], rs, RTOL_BF16, f"s_T g={g} head ({b},{h})")


@pytest.mark.parametrize("g", [2, 4])
def test_factors_state_form_resume(K, g):
    # two calls carrying the state equal one call; state-only mode as well
    c = S.prefill_case("factors_resume", 1, 3, 500, 64, 64, 64, seed=91 + g)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    T1 = 192
    o1, H1, s1 = K.prefill(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], chunk=64, return_state=True, factors=g)
    o2, H2, s2 = K.prefill(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], chunk=128, state=(H1, s1),
                           return_state=True, factors=g)
    Hs, ss = K.prefill(q, k, v, chunk=64, outputs=False, factors=g)
    ro = np.stack([O.prefill_factors_bruteforce(c.q[0, h], c.k[0, h], c.v[0, h], g, "concat") for h in range(3)])
    assert_close(host(torch.cat([o1, o2], dim=2))[0], ro, RTOL_BF16, "resumed o")
    for h in range(3):
        _, rH, rs = O.prefill_factors_recurrent(c.q[0, h], c.k[0, h], c.v[0, h], g, "concat")
        assert_close(host(H2)[0, h], rH, RTOL_BF16, "resumed H")
        assert_close(host(Hs)[0, h], rH, RTOL_BF16, "state-only H")
        assert_close(host(ss)[0, h], rs, RTOL_BF16, "state-only s")


def test_factors_state_form_one_factor_is_prefill(K):
    c = S.prefill_case("factors_one", 1, 2, 200, 64, 64, 64, seed=95)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    a = K.prefill(q, k, v, chunk=64)
    b = K.prefill(q, k, v, chunk=64, factors=1)
    assert torch.equal(a, b)


def test_factors_state_form_4x8x4096_full_size(K):
    # KATA-M2 on the main prefill workload: sampled rows and one head's state
    cfg = S.CONFIGS["prefill_4x8x4096"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    c = S.prefill_case("prefill_4x8x4096", B, H, T, cfg["d_qk"], cfg["d_v"], cfg["chunk"], cfg["seed"])
    o, HT, sT = K.prefill(dev(c.q), dev(c.k), dev(c.v), chunk=64, return_state=True, factors=2)
    go = host(o)
    rng = np.random.default_rng(6)
    for (b, h) in [(0, 0), (B - 1, H - 1)]:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, T - 1], rng.integers(0, T, 12)]))
        W = np.where(np.arange(T)[None, :] <= rows[:, None],
                     O.factor_weights(c.q[b, h][rows], c.k[b, h], 2, "concat"), 0.0)
        ref = (W @ c.v[b, h].astype(np.float64)) / W.sum(axis=1)[:, None]
        assert_close(go[b, h, rows], ref, RTOL_BF16, f"o rows head ({b},{h})")
    fk = O.phi_factors(c.k[1, 3], 2, "concat")
    assert_close(host(HT)[1, 3], fk.T @ c.v[1, 3].astype(np.float64), RTOL_BF16, "H_T head (1,3)")
    assert_close(host(sT)[1, 3], fk.sum(axis=0), RTOL_BF16, "s_T head (1,3)")


# ---- the concatenated lift on the float32 vector path (float32 inputs, any
# supported head size): float32 arithmetic throughout, so the fp32 bound

@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("B,H,T,dqk,dv,chunk,eps", [(1, 2, 100, 64, 64, 64, 0.0), (2, 3, 77, 32, 16, 32, 0.2),
                                                    (1, 2, 300, 16, 64, 128, 0.0), (1, 1, 1, 32, 32, 64, 0.0)])
def test_factors_f32_every_row(K, g, B, H, T, dqk, dv, chunk, eps):
    c = S.prefill_case("factors_f32", B, H, T, dqk, dv, chunk, seed=300 + g + T + dqk)
    f32 = lambda x: dev(x, torch.float32)
    o, HT, sT = K.prefill(f32(c.q), f32(c.k), f32(c.v), chunk=chunk, eps=eps, return_state=True, factors=g)
    torch.cuda.synchronize()
    assert HT.shape == (B, H, K.factor_phi_dim(dqk, g), dv)
    for b in range(B):
        for h in range(H):
            ro, rH, rs = O.prefill_factors_recurrent(c.q[b, h], c.k[b, h], c.v[b, h], g, "concat", eps=eps)
            assert_close(host(o)[b, h], ro, RTOL_F32, f"o g={g} head ({b},{h})")
            assert_close(host(HT)[b, h], rH, RTOL_F32, f"H_T g={g} head ({b},{h})")
            assert_close(host(sT)[b, h], rs, RTOL_F32, f"s_T g={g} head ({b},{h})")


@pytest.mark.parametrize("g", [2, 4])
def test_factors_f32_resume_and_bf16_out(K, g):
    # resuming from a carried state, and the bf16 output of float32 inputs
    c = S.prefill_case("factors_f32_resume", 1, 2, 260, 32, 32, 64, seed=77 + g)
    q, k, v = (dev(x, torch.float32) for x in (c.q, c.k, c.v))
    T1 = 100
    o1, H1, s1 = K.prefill(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], chunk=64, return_state=True, factors=g)
    o2 = K.prefill(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], chunk=32, state=(H1, s1), factors=g)
    ob = K.prefill(q, k, v, chunk=64, out_dtype=torch.bfloat16, factors=g)
    for h in range(2):
        ro = O.prefill_factors_bruteforce(c.q[0, h], c.k[0, h], c.v[0, h], g, "concat")
        assert_close(host(torch.cat([o1, o2], dim=2))[0, h], ro, RTOL_F32, f"resumed o head {h}")
        assert_close(host(ob)[0, h], ro, RTOL_BF16, f"bf16 out head {h}")


@pytest.mark.parametrize("g", [2, 4])
def test_factors_vector_path_bf16_inputs(K, g):
    # bf16 inputs with d_qk = 32 (not the matrix path): float32 arithmetic on
    # exact bf16 values, so the float32 bound against the oracle on the same
    # rounded inputs
    c = S.prefill_case("factors_vec_bf16", 1, 2, 150, 32, 64, 64, seed=510 + g)
    qb, kb, vb = (dev(x) for x in (c.q, c.k, c.v))
    o, HT, sT = K.prefill(qb, kb, vb, chunk=64, return_state=True, out_dtype=torch.float32, factors=g)
    torch.cuda.synchronize()
    q, k, v = host(qb), host(kb), host(vb)
    for h in range(2):
        ro, rH, rs = O.prefill_factors_recurrent(q[0, h], k[0, h], v[0, h], g, "concat")
        assert_close(host(o)[0, h], ro, RTOL_F32, f"o g={g} head {h}")
        assert_close(host(HT)[0, h], rH, RTOL_F32, f"H_T g={g} head {h}")
        assert_close(host(sT)[0, h], rs, RTOL_F32, f"s_T g={g} head {h}")


# ---- the summed lift (KATA-Sigma-g) through the chunked state form: the
# float32 vector path for float32 inputs and for head sizes other than 64
# (float32 arithmetic on exact inputs, so the float32 bound against the
# oracle's state form of the same lift); bf16 inputs with d_qk = d_v = 64 take
# the matrix-core kernel (tests further below, at the bf16 bound)

@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("B,H,T,dqk,dv,chunk,eps,dtype", [
    (1, 2, 100, 64, 64, 64, 0.0, torch.float32), (2, 3, 77, 32, 16, 32, 0.2, torch.float32),
    (1, 2, 300, 16, 64, 128, 0.0, torch.float32), (1, 1, 1, 32, 32, 64, 0.0, torch.float32),
    (1, 3, 97, 64, 32, 32, 0.1, torch.bfloat16), (1, 2, 70, 32, 64, 64, 0.0, torch.bfloat16)])
def test_factors_sum_state_form_every_row(K, g, B, H, T, dqk, dv, chunk, eps, dtype):
    c = S.prefill_case("factors_sum_state", B, H, T, dqk, dv, chunk, seed=600 + g + T + dqk)
    o, HT, sT = K.prefill(dev(c.q, dtype), dev(c.k, dtype), dev(c.v, dtype), chunk=chunk, eps=eps,
                          return_state=True, out_dtype=torch.float32, factors=g, factor_kind="sum")
    torch.cuda.synchronize()
    D = K.factor_phi_dim(dqk, g, "sum")
    assert D == (dqk // g) * (dqk // g + 1) // 2
    assert HT.shape == (B, H, D, dv) and sT.shape == (B, H, D)
    # the oracle sees the values the GPU read (bf16-rounded for bf16 inputs)
    q, k, v = (host(dev(x, dtype)) for x in (c.q, c.k, c.v))
    for b in range(B):
        for h in range(H):
            ro, rH, rs = O.prefill_factors_recurrent(q[b, h], k[b, h], v[b, h], g, "sum", eps=eps)
            assert_close(host(o)[b, h], ro, RTOL_F32, f"o g={g} head ({b},{h})")
            assert_close(host(HT)[b, h], rH, RTOL_F32, f"H_T g={g} head ({b},{h})")
            assert_close(host(sT)[b, h], rs, RTOL_F32, f"s_T g={g} head ({b},{h})")


@pytest.mark.parametrize("g", [2, 4])
def test_factors_sum_state_form_resume(K, g):
    # two calls carrying the summed lift's state equal one call, and equal the
    # closed-form definition sum_{i,j} (q_i . k_j)^2; state-only mode too
    c = S.prefill_case("factors_sum_resume", 1, 2, 400, 64, 64, 64, seed=640 + g)
    q, k, v = (dev(x, torch.float32) for x in (c.q, c.k, c.v))
    T1 = 150
    o1, H1, s1 = K.prefill(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], chunk=64, return_state=True, factors=g,
                           factor_kind="sum")
    o2 = K.prefill(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], chunk=128, state=(H1, s1), factors=g,
                   factor_kind="sum")
    Hs, ss = K.prefill(q, k, v, chunk=32, outputs=False, factors=g, factor_kind="sum")
    for h in range(2):
        ro = O.prefill_factors_bruteforce(c.q[0, h], c.k[0, h], c.v[0, h], g, "sum")
        assert_close(host(torch.cat([o1, o2], dim=2))[0, h], ro, RTOL_F32, f"resumed o head {h}")
        _, rH, rs = O.prefill_factors_recurrent(c.q[0, h], c.k[0, h], c.v[0, h], g, "sum")
        assert_close(host(Hs)[0, h], rH, RTOL_F32, f"state-only H head {h}")
        assert_close(host(ss)[0, h], rs, RTOL_F32, f"state-only s head {h}")


def test_factors_sum_one_factor_is_prefill(K):
    c = S.prefill_case("factors_sum_one", 1, 2, 120, 32, 32, 32, seed=660)
    q, k, v = (dev(x, torch.float32) for x in (c.q, c.k, c.v))
    a = K.prefill(q, k, v, chunk=32)
    b = K.prefill(q, k, v, chunk=32, factors=1, factor_kind="sum")
    assert torch.equal(a, b)


# ---- the summed lift on the matrix cores (bf16 inputs, d_qk = d_v = 64):
# float16 products of the staged inputs, float32 accumulation, so the bf16
# bound against the oracle's state form on the same rounded inputs

@pytest.mark.parametrize("g", [2, 4])
@pytest.mark.parametrize("B,H,chunk,T,eps", [(1, 3, 64, 50, 0.0), (2, 2, 128, 300, 0.0), (2, 10, 64, 130, 0.1),
                                              (1, 17, 32, 97, 0.0), (1, 2, 64, 1, 0.0)])
def test_factors_sum_matrix_path_every_row(K, g, B, H, chunk, T, eps):
    assert K.prefill_uses_matrix_cores(B, H, T, 64, 64, chunk)
    c = S.prefill_case("factors_sum_mfma", B, H, T, 64, 64, chunk, seed=700 + g + T)
    o, HT, sT = K.prefill(dev(c.q), dev(c.k), dev(c.v), chunk=chunk, eps=eps, return_state=True,
                          out_dtype=torch.float32, factors=g, factor_kind="sum")
    torch.cuda.synchronize()
    D = K.factor_phi_dim(64, g, "sum")
    assert HT.shape == (B, H, D, 64) and sT.shape == (B, H, D)
    for b in range(B):
        for h in range(H):
            ro, rH, rs = O.prefill_factors_recurrent(c.q[b, h], c.k[b, h], c.v[b, h], g, "sum", eps=eps)
            assert_close(host(o)[b, h], ro, RTOL_BF16, f"o g={g} head ({b},{h})")
            assert_close(host(HT)[b, h], rH, RTOL_BF16, f"H_T g={g} head ({b},{h})")
            assert_close(host(sT)[b, h], rs, RTOL_BF16, f"s_T g={g} head ({b},{h})")


@pytest.mark.parametrize("g", [2, 4])
def test_factors_sum_matrix_path_resume(K, g):
    # a state carried between calls (imported, exported) equals one call, and
    # equals the definition sum_{i,j} (q_i . k_j)^2; state-only mode too
    c = S.prefill_case("factors_sum_mfma_resume", 1, 3, 500, 64, 64, 64, seed=720 + g)
    q, k, v = dev(c.q), dev(c.k), dev(c.v)
    T1 = 192
    o1, H1, s1 = K.prefill(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], chunk=64, return_state=True, factors=g,
                           factor_kind="sum")
    o2, H2, s2 = K.prefill(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], chunk=128, state=(H1, s1),
                           return_state=True, factors=g, factor_kind="sum")
    Hs, ss = K.prefill(q, k, v, chunk=32, outputs=False, factors=g, factor_kind="sum")
    ro = np.stack([O.prefill_factors_bruteforce(c.q[0, h], c.k[0, h], c.v[0, h], g, "sum") for h in range(3)])
    assert_close(host(torch.cat([o1, o2], dim=2))[0], ro, RTOL_BF16, "resumed o")
    for h in range(3):
        _, rH, rs = O.prefill_factors_recurrent(c.q[0, h], c.k[0, h], c.v[0, h], g, "sum")
        assert_close(host(H2)[0, h], rH, RTOL_BF16, "resumed H")
        assert_close(host(s2)[0, h], rs, RTOL_BF16, "resumed s")
        assert_close(host(Hs)[0, h], rH, RTOL_BF16, "state-only H")
        assert_close(host(ss)[0, h], rs, RTOL_BF16, "state-only s")


def test_factors_sum_matrix_path_4x8x4096_full_size(K):
    # KATA-Sigma-2 on the main prefill workload: every row of two heads against
    # the oracle's state form, sampled rows of two more against the definition,
    # the final state of one head
    cfg = S.CONFIGS["prefill_4x8x4096"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    c = S.prefill_case("prefill_4x8x4096", B, H, T, cfg["d_qk"], cfg["d_v"], cfg["chunk"], cfg["seed"])
    o, HT, sT = K.prefill(dev(c.q), dev(c.k), dev(c.v), chunk=64, return_state=True, factors=2, factor_kind="sum")
    go, gH, gs = host(o), host(HT), host(sT)
    for (b, h) in [(0, 0), (B - 1, H - 1)]:
        ro, rH, rs = O.prefill_factors_recurrent(c.q[b, h], c.k[b, h], c.v[b, h], 2, "sum")
        assert_close(go[b, h], ro, RTOL_BF16, f"o head ({b},{h})")
        assert_close(gH[b, h], rH, RTOL_BF16, f"H_T head ({b},{h})")
        assert_close(gs[b, h], rs, RTOL_BF16, f"s_T head ({b},{h})")
    rng = np.random.default_rng(8)
    for (b, h) in [(1, 3), (2, 6)]:
        rows = np.unique(np.concatenate([[0, 1, 63, 64, T - 1], rng.integers(0, T, 12)]))
        W = np.where(np.arange(T)[None, :] <= rows[:, None],
                     O.factor_weights(c.q[b, h][rows], c.k[b, h], 2, "sum"), 0.0)
        ref = (W @ c.v[b, h].astype(np.float64)) / W.sum(axis=1)[:, None]
        assert_close(go[b, h, rows], ref, RTOL_BF16, f"o rows head ({b},{h})")
