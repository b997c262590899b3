"""GPU parity: every kernel behind the C ABI against the float64 oracle on the
same seeded inputs. Run on an MI355X with ``pytest -m gpu``.

Small cases cover every supported (d_qk, d_v, chunk), float32 and bf16
inputs, ragged tails, resumed state and the state-only mode, at sizes the
oracle finishes in seconds. The full-size workloads are checked on sampled
outputs (brute-force rows, sampled heads and head-states).

Tolerances (tests/tolerance.py): 1e-4 for float32 arithmetic paths, 2e-2
for bf16-input matrix-core paths and bf16 outputs; top-k sets exact outside
near-ties (relative boundary gap > 1e-5).
"""
import math

import numpy as np
import pytest

import oracle as O
from kernelized_linear_attention_02_amd import synth as S
from tests.tolerance import RTOL_BF16, RTOL_F32, TIE_REL, assert_close

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


def tdtype(case_dtype):
    return torch.bfloat16 if case_dtype == "bf16" else torch.float32


# ------------------------------------------------------------------ prefill

def test_tiny_f32_config(K):
    cfg = S.CONFIGS["tiny_f32"]
    c = S.prefill_case("tiny", cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], cfg["chunk"],
                       cfg["seed"], kind="tiny")
    o, HT, sT = K.prefill(dev(c.q), dev(c.k), dev(c.v), chunk=c.chunk, return_state=True)
    torch.cuda.synchronize()
    q, k, v = (x[0, 0].astype(np.float64) for x in (c.q, c.k, c.v))
    ob = O.prefill_bruteforce(q, k, v)
    orr, Hr, sr = O.prefill_recurrent(q, k, v)
    assert_close(host(o)[0, 0], ob, RTOL_F32, "o vs brute force")
    assert_close(host(o)[0, 0], orr, RTOL_F32, "o vs recurrent")
    assert_close(host(HT)[0, 0], Hr, RTOL_F32, "H_T")
    assert_close(host(sT)[0, 0], sr, RTOL_F32, "s_T")


@pytest.mark.parametrize("dqk,dv", [(16, 16), (16, 64), (32, 32), (64, 16), (64, 64)])
@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 77, 300])
def test_prefill_f32_shapes(K, dqk, dv, chunk, T):
    rng = np.random.default_rng([dqk, dv, chunk, T])
    B, H = 1, 2
    q = rng.standard_normal((B, H, T, dqk)).astype(np.float32) / math.sqrt(dqk)
    k = rng.standard_normal((B, H, T, dqk)).astype(np.float32) / math.sqrt(dqk)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    o, HT, sT = K.prefill(dev(q), dev(k), dev(v), chunk=chunk, return_state=True)
    ro, rH, rs = O.prefill(q, k, v, chunk=97)
    assert_close(host(o), ro, RTOL_F32, "o")
    assert_close(host(HT), rH, RTOL_F32, "H_T")
    assert_close(host(sT), rs, RTOL_F32, "s_T")


@pytest.mark.parametrize("chunk", [32, 64, 128])
@pytest.mark.parametrize("T", [50, 513])
def test_prefill_bf16_d64(K, chunk, T):
    c = S.prefill_case("small", 2, 2, T, 64, 64, chunk, seed=20 + T)
    o, HT, sT = K.prefill(dev(c.q, torch.bfloat16), dev(c.k, torch.bfloat16),
                          dev(c.v, torch.bfloat16), chunk=chunk, return_state=True)
    assert o.dtype == torch.bfloat16
    ro, rH, rs = O.prefill(c.q, c.k, c.v, chunk=256)
    assert_close(host(o), ro, RTOL_BF16, "o")
    assert_close(host(HT), rH, RTOL_BF16, "H_T")
    assert_close(host(sT), rs, RTOL_BF16, "s_T")
    # float32 outputs from the same bf16 inputs
    o32 = K.prefill(dev(c.q, torch.bfloat16), dev(c.k, torch.bfloat16), dev(c.v, torch.bfloat16),
                    chunk=chunk, out_dtype=torch.float32)
    assert o32.dtype == torch.float32
    assert_close(host(o32), ro, RTOL_BF16, "o (f32 out)")


@pytest.mark.parametrize("B,H,chunk,T", [(2, 10, 64, 150), (3, 8, 128, 260), (1, 17, 32, 97)])
def test_prefill_bf16_d64_many_heads(K, B, H, chunk, T):
    # more than 16 heads: the matrix path splits each head's features in 8
    # slices of two tile columns instead of 16 slices of one
    c = S.prefill_case("many", B, H, T, 64, 64, chunk, seed=40 + H)
    o, HT, sT = K.prefill(dev(c.q, torch.bfloat16), dev(c.k, torch.bfloat16),
                          dev(c.v, torch.bfloat16), chunk=chunk, return_state=True)
    ro, rH, rs = O.prefill(c.q, c.k, c.v, chunk=128)
    assert_close(host(o), ro, RTOL_BF16, "o")
    assert_close(host(HT), rH, RTOL_BF16, "H_T")
    assert_close(host(sT), rs, RTOL_BF16, "s_T")


def test_prefill_resume_and_state_only(K):
    rng = np.random.default_rng(31)
    T1, T2, d = 130, 90, 32
    q = rng.standard_normal((1, 3, T1 + T2, d)).astype(np.float32) / math.sqrt(d)
    k = rng.standard_normal((1, 3, T1 + T2, d)).astype(np.float32) / math.sqrt(d)
    v = rng.standard_normal((1, 3, T1 + T2, d)).astype(np.float32)
    Q, Kk, V = dev(q), dev(k), dev(v)
    o, H, s = K.prefill(Q, Kk, V, chunk=64, return_state=True)
    o1, H1, s1 = K.prefill(Q[:, :, :T1], Kk[:, :, :T1], V[:, :, :T1], chunk=32, return_state=True)
    o2, H2, s2 = K.prefill(Q[:, :, T1:], Kk[:, :, T1:], V[:, :, T1:], chunk=128, state=(H1, s1),
                           return_state=True)
    assert_close(host(torch.cat([o1, o2], dim=2)), host(o), RTOL_F32, "resumed o")
    assert_close(host(H2), host(H), RTOL_F32, "resumed H")
    Hs, ss = K.prefill(Q, Kk, V, chunk=64, outputs=False)
    assert_close(host(Hs), host(H), RTOL_F32, "state-only H")
    assert_close(host(ss), host(s), RTOL_F32, "state-only s")
    # resume in place: H_T aliases H0
    ro, rH, rs = O.prefill(q, k, v, chunk=50)
    assert_close(host(H), rH, RTOL_F32, "H vs oracle")


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_prefill_bf16_resume_and_state_only(K, chunk):
    # resumed bf16 prefill through the matrix-core path equals one call
    c = S.prefill_case("resume", 1, 3, 700, 64, 64, chunk, seed=33)
    Q, Kk, V = (dev(x, torch.bfloat16) for x in (c.q, c.k, c.v))
    T1 = 300
    o1, H1, s1 = K.prefill(Q[:, :, :T1], Kk[:, :, :T1], V[:, :, :T1], chunk=chunk, return_state=True)
    o2, H2, s2 = K.prefill(Q[:, :, T1:], Kk[:, :, T1:], V[:, :, T1:], chunk=chunk, state=(H1, s1),
                           return_state=True)
    ro, rH, rs = O.prefill(c.q, c.k, c.v, chunk=100)
    assert_close(host(torch.cat([o1, o2], dim=2)), ro, RTOL_BF16, "resumed o")
    assert_close(host(H2), rH, RTOL_BF16, "resumed H")
    assert_close(host(s2), rs, RTOL_BF16, "resumed s")
    Hs, ss = K.prefill(Q, Kk, V, chunk=chunk, outputs=False)
    assert_close(host(Hs), rH, RTOL_BF16, "state-only H")
    assert_close(host(ss), rs, RTOL_BF16, "state-only s")


def test_prefill_matrix_path_selected(K):
    assert K.prefill_uses_matrix_cores(B=4, H=8, T=4096, d_qk=64, d_v=64, chunk=64)
    assert not K.prefill_uses_matrix_cores(d_qk=32, d_v=32)
    assert not K.prefill_uses_matrix_cores(dtype=0)


def test_prefill_degenerate_inputs(K):
    # zero queries: every denominator is 0 and the output is 0; eps > 0 keeps it 0
    T, d = 70, 16
    z = torch.zeros((1, 1, T, d), device="cuda")
    kk = torch.randn((1, 1, T, d), device="cuda")
    vv = torch.randn((1, 1, T, d), device="cuda")
    assert torch.all(K.prefill(z, kk, vv, chunk=32) == 0)
    assert torch.all(K.prefill(z, kk, vv, chunk=32, eps=1e-3) == 0)
    # a single token returns its own value
    q1 = torch.randn((1, 2, 1, 64), device="cuda")
    k1 = torch.randn((1, 2, 1, 64), device="cuda")
    v1 = torch.randn((1, 2, 1, 64), device="cuda")
    assert_close(host(K.prefill(q1, k1, v1, chunk=64)), host(v1), RTOL_F32, "T=1")


def _prefill_full(K, name, brute_rows_per_head):
    """The workload as configured, every output row and the final state of
    every head against the oracle's chunked form (its own chunk of 256), plus
    seeded rows against the brute-force definition."""
    cfg = S.CONFIGS[name]
    c = S.prefill_case(name, cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], cfg["chunk"],
                       cfg["seed"], threads=16)
    o, HT, sT = K.prefill(dev(c.q, torch.bfloat16), dev(c.k, torch.bfloat16),
                          dev(c.v, torch.bfloat16), chunk=c.chunk, return_state=True)
    torch.cuda.synchronize()
    go, gH, gs = o.float().cpu().numpy(), HT.cpu().numpy(), sT.cpu().numpy()
    del o, HT, sT
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    rng = np.random.default_rng(99)
    worst = dict(o=0.0, H=0.0, s=0.0, brute=0.0)
    for b in range(B):
        for h in range(H):
            ro, rH, rs = O.prefill_chunked(c.q[b, h], c.k[b, h], c.v[b, h], chunk=256)
            worst["o"] = max(worst["o"], assert_close(go[b, h], ro, RTOL_BF16, f"o of head ({b},{h})")["max_scaled"])
            worst["H"] = max(worst["H"], assert_close(gH[b, h], rH, RTOL_BF16, f"H_T of head ({b},{h})")["max_scaled"])
            worst["s"] = max(worst["s"], assert_close(gs[b, h], rs, RTOL_BF16, f"s_T of head ({b},{h})")["max_scaled"])
            rows = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, brute_rows_per_head)]))
            ref = O.prefill_bruteforce_rows(c.q[b, h], c.k[b, h], c.v[b, h], rows)
            rep = assert_close(go[b, h, rows], ref, RTOL_BF16, f"brute-force rows of head ({b},{h})")
            worst["brute"] = max(worst["brute"], rep["max_scaled"])
    print(f"[parity] {name}: worst scaled error {worst}", flush=True)


def test_prefill_4x8x4096_full_size(K):
    _prefill_full(K, "prefill_4x8x4096", 32)


def test_prefill_1x16x65536_full_size(K):
    _prefill_full(K, "prefill_1x16x65536", 64)


# ------------------------------------------------------------------ quadratic form

def _bruteforce_heads(q, k, v, eps=0.0):
    B, H = q.shape[:2]
    return np.stack([np.stack([O.prefill_bruteforce(q[b, h], k[b, h], v[b, h], eps=eps) for h in range(H)])
                     for b in range(B)])


@pytest.mark.parametrize("T", [1, 5, 64, 127, 128, 129, 300, 1000])
def test_prefill_quadratic_shapes(K, T):
    # against the float64 brute-force definition (every row), bf16 and f32 outputs
    c = S.prefill_case("quad", 1, 3, T, 64, 64, 64, seed=120 + T)
    Q, Kk, V = (dev(x, torch.bfloat16) for x in (c.q, c.k, c.v))
    ref = _bruteforce_heads(c.q, c.k, c.v)
    o = K.prefill_quadratic(Q, Kk, V)
    assert o.dtype == torch.bfloat16
    assert_close(host(o), ref, RTOL_BF16, f"quadratic o, T={T}")
    o32 = K.prefill_quadratic(Q, Kk, V, out_dtype=torch.float32, eps=0.3)
    assert o32.dtype == torch.float32
    assert_close(host(o32), _bruteforce_heads(c.q, c.k, c.v, eps=0.3), RTOL_BF16,
                 f"quadratic o, T={T}, eps")


def test_prefill_quadratic_degenerate(K):
    # zero queries: every denominator is 0 and the output is 0 (also with eps);
    # a single token returns its own value
    T = 200
    z = torch.zeros((1, 2, T, 64), device="cuda", dtype=torch.bfloat16)
    kk = torch.randn((1, 2, T, 64), device="cuda").to(torch.bfloat16)
    vv = torch.randn((1, 2, T, 64), device="cuda").to(torch.bfloat16)
    assert torch.all(K.prefill_quadratic(z, kk, vv) == 0)
    assert torch.all(K.prefill_quadratic(z, kk, vv, eps=1e-3) == 0)
    q1 = torch.randn((2, 3, 1, 64), device="cuda").to(torch.bfloat16)
    k1 = torch.randn((2, 3, 1, 64), device="cuda").to(torch.bfloat16)
    v1 = torch.randn((2, 3, 1, 64), device="cuda").to(torch.bfloat16)
    assert_close(host(K.prefill_quadratic(q1, k1, v1, out_dtype=torch.float32)), host(v1), RTOL_BF16, "T=1")


def test_prefill_quadratic_4x8x4096_full_size(K):
    # the headline workload through the quadratic form: sampled rows against the
    # brute force, and every row against the chunked matrix-core path
    cfg = S.CONFIGS["prefill_4x8x4096"]
    c = S.prefill_case("prefill_4x8x4096", cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"],
                       cfg["chunk"], cfg["seed"])
    Q, Kk, V = (dev(x, torch.bfloat16) for x in (c.q, c.k, c.v))
    oq = K.prefill_quadratic(Q, Kk, V, out_dtype=torch.float32)
    oc = K.prefill(Q, Kk, V, chunk=cfg["chunk"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    go = oq.cpu().numpy()
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    rng = np.random.default_rng(98)
    for b in range(B):
        for h in range(H):
            rows = np.unique(np.concatenate([[0, 1, T - 1], rng.integers(0, T, 16)]))
            ref = O.prefill_bruteforce_rows(c.q[b, h], c.k[b, h], c.v[b, h], rows)
            assert_close(go[b, h, rows], ref, RTOL_BF16, f"quadratic rows of head ({b},{h})")
    assert_close(go, oc.cpu().numpy(), 2 * RTOL_BF16, "quadratic vs chunked")


# ------------------------------------------------------------------ decode + SRE

def _initial_state(K, case):
    pk = dev(case.prefix_k)[None]
    pv = dev(case.prefix_v)[None]
    H, s = K.prefill(pk, pk, pv, chunk=64, outputs=False)
    return H[0].contiguous(), s[0].contiguous()


def test_decode_step_small(K):
    case = S.decode_case(6, d=64, T0=200, steps=5, seed=41)
    H, s = _initial_state(K, case)
    rH0 = np.stack([O.phi(case.prefix_k[n]).T @ case.prefix_v[n].astype(np.float64) for n in range(6)])
    assert_close(host(H), rH0, RTOL_F32, "initial state")
    rH, rs = rH0.copy(), np.stack([O.phi(case.prefix_k[n]).sum(0) for n in range(6)])
    for t in range(5):
        o = K.decode_step(H, s, dev(case.q[t]), dev(case.k[t]), dev(case.v[t]))
        ro = np.zeros((6, 64))
        for n in range(6):
            ro[n], rH[n], rs[n] = O.decode_step(rH[n], rs[n], case.q[t, n], case.k[t, n], case.v[t, n])
        assert_close(host(o), ro, RTOL_F32, f"decode o step {t}")
    assert_close(host(H), rH, RTOL_F32, "decode H")
    assert_close(host(s), rs, RTOL_F32, "decode s")


def test_sre_zero_for_signed_basis_keys(K):
    # phi(e_i).phi(e_j) = delta_ij: recall of each stored pair is exact on the GPU too
    d = 64
    idx = np.array([3, 17, 40, 63, 0, 9])
    keys = np.eye(d, dtype=np.float32)[idx] * np.array([1, -1, 1, -1, 1, 1], np.float32)[:, None]
    vals = np.random.default_rng(5).standard_normal((len(idx), d)).astype(np.float32)
    H, s = K.prefill(dev(keys)[None, None], dev(keys)[None, None], dev(vals)[None, None], chunk=32,
                     outputs=False)
    r = K.sre_select(H[0], s[0], dev(keys)[None], dev(vals)[None], top_k=3)
    assert np.all(host(r["scores"]) == 0.0)
    assert sorted(host(r["sel"]).astype(int)[0].tolist()) == [0, 1, 2]  # ties -> lowest index


@pytest.mark.parametrize("n_cand,top_k", [(64, 16), (100, 7), (256, 128), (5, 5)])
def test_sre_select_against_oracle(K, n_cand, top_k):
    rng = np.random.default_rng(n_cand)
    N, d = 5, 64
    pk = rng.standard_normal((N, 300, d)).astype(np.float32) / 8
    pv = rng.standard_normal((N, 300, d)).astype(np.float32)
    H, s = K.prefill(dev(pk)[None], dev(pk)[None], dev(pv)[None], chunk=128, outputs=False)
    ck = rng.standard_normal((N, n_cand, d)).astype(np.float32) / 8
    cv = rng.standard_normal((N, n_cand, d)).astype(np.float32)
    r = K.sre_select(H[0], s[0], dev(ck), dev(cv), top_k=top_k, gather=True)
    for n in range(N):
        fk = O.phi(pk[n])
        rs = O.sre(fk.T @ pv[n].astype(np.float64), fk.sum(0), ck[n], cv[n])
        assert_close(host(r["scores"])[n], rs, RTOL_F32, f"scores head {n}")
        sel = host(r["sel"]).astype(int)[n]
        assert O.near_tie_ok(rs, sel, top_k, TIE_REL), f"selection head {n}"
        # order within sel follows the GPU's own scores (descending, index ascending)
        gs = host(r["scores"])[n]
        assert list(sel) == list(O.select_topk(gs, top_k))
        np.testing.assert_array_equal(host(r["sel_k"])[n], ck[n][sel])
        np.testing.assert_array_equal(host(r["sel_v"])[n], cv[n][sel])


@pytest.mark.parametrize("n_cand,top_k", [(1, 1), (17, 4), (33, 33), (48, 12)])
@pytest.mark.parametrize("with_scores,gather", [(True, True), (False, False)])
def test_sre_select_matrix_path_shapes(K, n_cand, top_k, with_scores, gather):
    # d = 64 with at most 64 candidates runs on the matrix cores (split bf16)
    rng = np.random.default_rng(1000 + n_cand)
    N, d = 7, 64
    pk = rng.standard_normal((N, 200, d)).astype(np.float32) / 8
    pv = rng.standard_normal((N, 200, d)).astype(np.float32)
    H, s = K.prefill(dev(pk)[None], dev(pk)[None], dev(pv)[None], chunk=64, outputs=False)
    ck = rng.standard_normal((N, n_cand, d)).astype(np.float32) / 8
    ck[0, 0] = 0.0  # zero key: denominator 0, prediction 0, score ||v||^2
    cv = rng.standard_normal((N, n_cand, d)).astype(np.float32)
    H0, s0 = H.clone(), s.clone()
    r = K.sre_select(H[0], s[0], dev(ck), dev(cv), top_k=top_k, scores=with_scores, gather=gather)
    torch.cuda.synchronize()
    assert torch.equal(H, H0) and torch.equal(s, s0), "scoring must not write the state"
    for n in range(N):
        fk = O.phi(pk[n])
        rs = O.sre(fk.T @ pv[n].astype(np.float64), fk.sum(0), ck[n], cv[n])
        if with_scores:
            assert_close(host(r["scores"])[n], rs, RTOL_F32, f"scores head {n}")
        sel = host(r["sel"]).astype(int)[n]
        assert len(set(sel.tolist())) == top_k and sel.min() >= 0 and sel.max() < n_cand
        assert O.near_tie_ok(rs, sel, top_k, TIE_REL), f"selection head {n}"
        if gather:
            np.testing.assert_array_equal(host(r["sel_k"])[n], ck[n][sel])
            np.testing.assert_array_equal(host(r["sel_v"])[n], cv[n][sel])
    if with_scores:
        assert host(r["scores"])[0, 0] == pytest.approx(float(np.sum(cv[0, 0].astype(np.float64) ** 2)),
                                                         rel=1e-6)


@pytest.mark.parametrize("dtype,out_dtype,eps", [("f32", "f32", 0.0), ("bf16", "bf16", 0.0),
                                                 ("f32", "f32", 0.25)])
def test_decode_step_with_selection_matrix_path(K, dtype, out_dtype, eps):
    rng = np.random.default_rng(77)
    N, d, n_cand, top_k = 9, 64, 40, 9
    pk = rng.standard_normal((N, 150, d)).astype(np.float32) / 8
    pv = rng.standard_normal((N, 150, d)).astype(np.float32)
    H, s = K.prefill(dev(pk)[None], dev(pk)[None], dev(pv)[None], chunk=32, outputs=False)
    H, s = H[0].contiguous(), s[0].contiguous()
    q = rng.standard_normal((N, d)).astype(np.float32) / 8
    k = rng.standard_normal((N, d)).astype(np.float32) / 8
    v = rng.standard_normal((N, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (S.round_to_bf16(x) for x in (q, k, v))
    ck = rng.standard_normal((N, n_cand, d)).astype(np.float32) / 8
    cv = rng.standard_normal((N, n_cand, d)).astype(np.float32)
    tt = tdtype(dtype)
    o, r = K.decode_step(H, s, dev(q, tt), dev(k, tt), dev(v, tt), eps=eps, out_dtype=tdtype(out_dtype),
                         cand_k=dev(ck), cand_v=dev(cv), top_k=top_k, gather=True)
    torch.cuda.synchronize()
    rtol_o = RTOL_BF16 if out_dtype == "bf16" else RTOL_F32
    for n in range(N):
        fk = O.phi(pk[n])
        rH, rs = fk.T @ pv[n].astype(np.float64), fk.sum(0)
        ro, rH, rs = O.decode_step(rH, rs, q[n], k[n], v[n], eps=eps)
        assert_close(host(o)[n], ro, rtol_o, f"o head {n}")
        assert_close(host(H)[n], rH, RTOL_F32, f"H head {n}")
        assert_close(host(s)[n], rs, RTOL_F32, f"s head {n}")
        rsc = O.sre(rH, rs, ck[n], cv[n], eps=eps)
        assert_close(host(r["scores"])[n], rsc, RTOL_F32, f"scores head {n}")
        sel = host(r["sel"]).astype(int)[n]
        assert O.near_tie_ok(rsc, sel, top_k, TIE_REL), f"selection head {n}"
        np.testing.assert_array_equal(host(r["sel_k"])[n], ck[n][sel])


@pytest.mark.parametrize("dtype,out_dtype,eps,n_cand,top_k", [
    ("f32", "f32", 0.0, 40, 9), ("bf16", "bf16", 0.0, 64, 16), ("f32", "f32", 0.25, 16, 3),
    ("bf16", "f32", 0.1, 33, 33)])
def test_decode_deferred_with_selection(K, dtype, out_dtype, eps, n_cand, top_k):
    """Deferred folds over 11 tokens (a fold at the eighth, a flush of three
    at the end), with fresh candidates at every token: o, scores, selections
    and gathered rows of every token against the oracle's recurrence, and the
    flushed state."""
    rng = np.random.default_rng(79 + n_cand)
    N, d, steps = 7, 64, 11
    pk = rng.standard_normal((N, 120, d)).astype(np.float32) / 8
    pv = rng.standard_normal((N, 120, d)).astype(np.float32)
    H, s = K.prefill(dev(pk)[None], dev(pk)[None], dev(pv)[None], chunk=32, outputs=False)
    H, s = H[0].contiguous(), s[0].contiguous()
    rH = [O.phi(pk[n]).T @ pv[n].astype(np.float64) for n in range(N)]
    rs = [O.phi(pk[n]).sum(0) for n in range(N)]
    tt = tdtype(dtype)
    rtol_o = RTOL_BF16 if out_dtype == "bf16" else RTOL_F32
    step = _Stepper(K, N, True)
    for t in range(steps):
        q, k, v = (rng.standard_normal((N, d)).astype(np.float32) / f for f in (8, 8, 1))
        if dtype == "bf16":
            q, k, v = (S.round_to_bf16(x) for x in (q, k, v))
        ck = rng.standard_normal((N, n_cand, d)).astype(np.float32) / 8
        cv = rng.standard_normal((N, n_cand, d)).astype(np.float32)
        o, r = step(H, s, dev(q, tt), dev(k, tt), dev(v, tt), eps=eps, out_dtype=tdtype(out_dtype),
                    cand_k=dev(ck), cand_v=dev(cv), top_k=top_k, gather=True)
        torch.cuda.synchronize()
        go, gsc, gsel, gsk = host(o), host(r["scores"]), host(r["sel"]).astype(int), host(r["sel_k"])
        for n in range(N):
            ro, rH[n], rs[n] = O.decode_step(rH[n], rs[n], q[n], k[n], v[n], eps=eps)
            assert_close(go[n], ro, rtol_o, f"o token {t} head {n}")
            rsc = O.sre(rH[n], rs[n], ck[n], cv[n], eps=eps)
            assert_close(gsc[n], rsc, RTOL_F32, f"scores token {t} head {n}")
            assert O.near_tie_ok(rsc, gsel[n], top_k, TIE_REL), f"selection token {t} head {n}"
            np.testing.assert_array_equal(gsk[n], ck[n][gsel[n]])
    assert step.n_pend == steps % K.decode_pending_period()
    step.finish(H, s)
    torch.cuda.synchronize()
    for n in range(N):
        assert_close(host(H)[n], rH[n], RTOL_F32, f"H head {n}")
        assert_close(host(s)[n], rs[n], RTOL_F32, f"s head {n}")


def _oracle_chain_check(gpu, H, s, H0s, s0s, inputs, cache0_k, cache0_v, top, check_ids):
    """Each checked head-state's oracle chain against what the GPU recorded,
    following the GPU's selections through near-ties (rule R17)."""
    Hh, sh = host(H), host(s)
    steps = len(gpu["o"])
    for j, n in enumerate(check_ids):
        bad = []

        def choose(tau, sc, sel, j=j):
            g = gpu["sel"][tau][j]
            if not O.near_tie_ok(sc, g, top, TIE_REL):
                bad.append(tau)
            return g
        q, k, v, fk, fv = (np.stack([x[i][j] for i in range(steps)]) for x in inputs)
        ref = O.decode_sre_chain(H0s[j], s0s[j], q, k, v, fk, fv, cache0_k[j], cache0_v[j], top, choose=choose)
        assert not bad, f"head-state {n}: selection differs outside near-ties at steps {bad}"
        assert_close(np.array([x[j] for x in gpu["o"]]), ref["o"], RTOL_F32, f"o of head-state {n}")
        assert_close(np.array([x[j] for x in gpu["scores"]]), ref["scores"], RTOL_F32,
                     f"scores of head-state {n}")
        assert_close(Hh[n], ref["H"], RTOL_F32, f"H of head-state {n}")
        assert_close(sh[n], ref["s"], RTOL_F32, f"s of head-state {n}")


class _Stepper:
    """decode_step, or decode_step_deferred with its pending slots (the
    count advances by one per token and wraps when the call folds)."""

    def __init__(self, K, N, deferred):
        self.K, self.deferred, self.n_pend = K, deferred, 0
        if deferred:
            self.pk, self.pv = K.decode_pending_slots(N)
            # slots above n_pend are ignored: fill them with values that would show
            self.pk.fill_(7.0)
            self.pv.fill_(-3.0)

    def __call__(self, H, s, q, k, v, **kw):
        if not self.deferred:
            return self.K.decode_step(H, s, q, k, v, **kw)
        r = self.K.decode_step_deferred(H, s, self.pk, self.pv, self.n_pend, q, k, v, **kw)
        self.n_pend = (self.n_pend + 1) % self.K.decode_pending_period()
        return r

    def finish(self, H, s):
        if self.deferred:
            self.K.decode_flush(H, s, self.pk, self.pv, self.n_pend)
            self.n_pend = 0


def _decode_chain(K, case, steps, check_ids, deferred=False):
    """Run the decode + selection chain on the GPU for all head-states and
    compare the head-states ``check_ids`` with the oracle."""
    N, d, top = case.N, case.d, case.top_k
    H, s = _initial_state(K, case)
    cache_k = dev(case.cache0_k)
    cache_v = dev(case.cache0_v)
    gpu = dict(o=[], scores=[], sel=[])
    step = _Stepper(K, N, deferred)
    for t in range(steps):
        cand_k = torch.cat([cache_k, dev(case.fresh_k[t])], dim=1)
        cand_v = torch.cat([cache_v, dev(case.fresh_v[t])], dim=1)
        o, r = step(H, s, dev(case.q[t]), dev(case.k[t]), dev(case.v[t]), cand_k=cand_k,
                    cand_v=cand_v, top_k=top, gather=True)
        cache_k, cache_v = r["sel_k"], r["sel_v"]
        gpu["o"].append(host(o)[check_ids])
        gpu["scores"].append(host(r["scores"])[check_ids])
        gpu["sel"].append(host(r["sel"]).astype(int)[check_ids])
    step.finish(H, s)
    torch.cuda.synchronize()
    H0s, s0s = [], []
    for n in check_ids:
        fk = O.phi(case.prefix_k[n])
        H0s.append(fk.T @ case.prefix_v[n].astype(np.float64))
        s0s.append(fk.sum(0))
    inputs = [[x[t][check_ids] for t in range(steps)] for x in (case.q, case.k, case.v, case.fresh_k, case.fresh_v)]
    _oracle_chain_check(gpu, H, s, H0s, s0s, inputs, case.cache0_k[check_ids], case.cache0_v[check_ids], top,
                        check_ids)


@pytest.mark.parametrize("deferred", [False, True])
def test_decode_chain_small(K, deferred):
    case = S.decode_case(8, d=64, T0=256, steps=12, seed=43)
    _decode_chain(K, case, 12, list(range(8)), deferred)


@pytest.mark.parametrize("steps", [1, 7, 8, 9, 20])
def test_decode_deferred_without_selection(K, steps):
    """Deferred folds with no candidates: every token's o, and the state after
    a flush at any point of the slot cycle, against the oracle's recurrence."""
    N, d = 5, 64
    case = S.decode_case(N, d=d, T0=64, steps=steps, seed=44)
    H, s = _initial_state(K, case)
    step = _Stepper(K, N, True)
    outs = [host(step(H, s, dev(case.q[t]), dev(case.k[t]), dev(case.v[t]))) for t in range(steps)]
    step.finish(H, s)
    torch.cuda.synchronize()
    for n in range(N):
        fk = O.phi(case.prefix_k[n])
        Hr, sr = fk.T @ case.prefix_v[n].astype(np.float64), fk.sum(0)
        ref = []
        for t in range(steps):
            o, Hr, sr = O.decode_step(Hr, sr, case.q[t][n], case.k[t][n], case.v[t][n])
            ref.append(o)
        assert_close(np.array([x[n] for x in outs]), np.array(ref), RTOL_F32, f"o of head-state {n}")
        assert_close(host(H)[n], Hr, RTOL_F32, f"H of head-state {n}")
        assert_close(host(s)[n], sr, RTOL_F32, f"s of head-state {n}")


@pytest.mark.parametrize("deferred", [False, True])
def test_decode_sre_4096x128_full_chain(K, deferred):
    """The decode workload as configured: 4096 head-states, a 2048-token
    prefix, 128 steps of update, readout, scoring of 16 cached + 48 fresh
    candidates and top-16 selection, gathered into the next step's candidate
    slab as the benchmark runs it. 64 seeded head-states are compared with
    the oracle at every step (o, scores, selected sets) and at the end (H, s);
    their initial state too."""
    cfg = S.CONFIGS["decode_sre_4096x128"]
    N, d, T0, steps, top, nf = cfg["N"], cfg["d"], cfg["T0"], cfg["steps"], cfg["top_k"], cfg["n_fresh"]
    stream = S.DecodeStream(N, d=d, T0=T0, top_k=top, n_fresh=nf, seed=cfg["seed"], threads=16)
    check = sorted(set(np.random.default_rng(7).choice(np.arange(1, N - 1), 62, replace=False).tolist())
                   | {0, N - 1})
    pk = dev(stream.prefix_k)[None]
    pv = dev(stream.prefix_v)[None]
    H, s = K.prefill(pk, pk, pv, chunk=64, outputs=False)
    H, s = H[0].contiguous(), s[0].contiguous()
    del pk, pv
    H0s, s0s = [], []
    for n in check:
        fk = O.phi(stream.prefix_k[n])
        H0s.append(fk.T @ stream.prefix_v[n].astype(np.float64))
        s0s.append(fk.sum(0))
    torch.cuda.synchronize()
    assert_close(host(H)[check], np.stack(H0s), RTOL_F32, "initial H")
    assert_close(host(s)[check], np.stack(s0s), RTOL_F32, "initial s")
    stream.drop_prefix()
    n_cand = top + nf
    ck = torch.empty((2, N, n_cand, d), device="cuda")
    cv = torch.empty((2, N, n_cand, d), device="cuda")
    ck[0, :, :top] = dev(stream.cache0_k)
    cv[0, :, :top] = dev(stream.cache0_v)
    o = torch.empty((N, d), device="cuda")
    sc = torch.empty((N, n_cand), device="cuda")
    sel = torch.empty((N, top), dtype=torch.int32, device="cuda")
    gpu = dict(o=[], scores=[], sel=[])
    inputs = [[], [], [], [], []]
    step = _Stepper(K, N, deferred)
    for t in range(steps):
        cur, nxt = t & 1, (t + 1) & 1
        q, k, v, fk, fv = stream.next_step()
        ck[cur, :, top:] = dev(fk)
        cv[cur, :, top:] = dev(fv)
        step(H, s, dev(q), dev(k), dev(v), cand_k=ck[cur], cand_v=cv[cur], top_k=top, gather=True,
             out=dict(o=o, scores=sc, sel=sel, sel_k=ck[nxt], sel_v=cv[nxt], sel_stride=n_cand))
        gpu["o"].append(host(o)[check])
        gpu["scores"].append(host(sc)[check])
        gpu["sel"].append(host(sel).astype(int)[check])
        for lst, x in zip(inputs, (q, k, v, fk, fv)):
            lst.append(x[check])
    step.finish(H, s)
    torch.cuda.synchronize()
    _oracle_chain_check(gpu, H, s, H0s, s0s, inputs, stream.cache0_k[check], stream.cache0_v[check], top, check)


# ------------------------------------------------------------------ hybrid

def _hybrid_check(K, c, heads, dtype, rtol, eps=0.0, out_dtype=None, aux=False):
    B, H, T, d = c.q.shape
    scale = 1.0 / math.sqrt(d)
    args = (dev(c.q, dtype), dev(c.k, dtype), dev(c.v, dtype), c.window, c.cache_size, c.refresh, scale)
    kw = dict(eps=eps, return_state=True, return_cache=True, return_trace=True, out_dtype=out_dtype)
    o, extra = K.hybrid_prefill(*args, **kw)
    if aux:
        # readouts on a second stream of the caller's: the same kernels, so
        # the same bits as the one-stream call
        side = torch.cuda.Stream()
        o2, extra2 = K.hybrid_prefill(*args, **kw, aux_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(o2, o), "two-stream outputs differ from one-stream outputs"
        for key in ("H", "s", "cache", "trace"):
            assert torch.equal(extra2[key], extra[key]), f"two-stream {key} differs"
    torch.cuda.synchronize()
    go, gH, gs = host(o), host(extra["H"]), host(extra["s"])
    gc = extra["cache"].cpu().numpy()
    gt = extra["trace"].cpu().numpy()
    for (b, h) in heads:
        bad = []

        def choose(blk, ids, sc, keep, b=b, h=h):
            g = [x for x in gt[b, h, blk].tolist() if x >= 0]
            pos = [int(np.nonzero(ids == x)[0][0]) for x in g if x in ids]
            if len(pos) != len(g) or not O.near_tie_ok(sc, pos, c.cache_size, TIE_REL):
                bad.append(blk)
                return keep
            return np.array(g)
        ref = O.hybrid_prefill(c.q[b, h], c.k[b, h], c.v[b, h], c.window, c.cache_size, c.refresh,
                               scale, eps=eps, choose=choose)
        assert not bad, f"head ({b},{h}): selections differ outside near-ties at blocks {bad[:5]}"
        nblk = gt.shape[2]
        for blk in range(nblk):
            if blk not in ref["trace"]:
                assert np.all(gt[b, h, blk] == -1)
        assert_close(go[b, h], ref["o"], rtol, f"hybrid o head ({b},{h})")
        assert_close(gH[b, h], ref["H"], max(rtol, RTOL_F32), f"hybrid H head ({b},{h})")
        assert_close(gs[b, h], ref["s"], max(rtol, RTOL_F32), f"hybrid s head ({b},{h})")
        want_cache = ref["cache"] + [-1] * (c.cache_size - len(ref["cache"]))
        assert gc[b, h].tolist() == want_cache


@pytest.mark.parametrize("d,W,lam,R,T", [(16, 32, 8, 16, 300), (64, 64, 16, 16, 410),
                                         (32, 48, 20, 8, 257), (64, 128, 64, 64, 700),
                                         (64, 96, 32, 64, 2100)])
def test_hybrid_small_bf16(K, d, W, lam, R, T):
    c = S.hybrid_case("small", 1, 2, T, d, W, lam, R, seed=60 + d + T, dup_frac=0.1)
    _hybrid_check(K, c, [(0, 0), (0, 1)], torch.bfloat16, RTOL_BF16)


@pytest.mark.parametrize("W,lam,R,T,H,eps,out", [
    (32, 0, 16, 200, 2, 0.0, torch.bfloat16),     # empty cache: every evicted pair folds
    (0, 16, 16, 190, 3, 0.0, torch.bfloat16),     # no window, three heads, ragged last block
    (64, 128, 128, 1000, 2, 0.0, torch.float32),  # largest cache + refresh (256 candidates)
    (40, 24, 7, 333, 3, 0.5, torch.float32),      # odd refresh, eps > 0, float32 output
])
def test_hybrid_matrix_path_edge_cases(K, W, lam, R, T, H, eps, out):
    # d = 64 with bf16 inputs takes the matrix-core path (fragment scorer,
    # counting selection), on one stream and with the readouts on a second
    c = S.hybrid_case("edge", 1, H, T, 64, W, lam, R, seed=90 + T + R, dup_frac=0.1)
    _hybrid_check(K, c, [(0, h) for h in range(H)], torch.bfloat16, RTOL_BF16, eps=eps, out_dtype=out,
                  aux=True)


def test_hybrid_special_cases_f32(K):
    # cache_size >= T and window >= T: plain causal softmax
    rng = np.random.default_rng(70)
    T, d = 150, 16
    q = rng.standard_normal((1, 1, T, d)).astype(np.float32) / 4
    k = rng.standard_normal((1, 1, T, d)).astype(np.float32) / 4
    v = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    scale = 0.25
    o = K.hybrid_prefill(dev(q), dev(k), dev(v), window=1000, cache_size=8, refresh=16,
                         softmax_scale=scale)
    ref = O.hybrid_prefill(q[0, 0], k[0, 0], v[0, 0], 1000, 8, 16, scale)["o"]
    assert_close(host(o)[0, 0], ref, RTOL_F32, "window >= T")
    # cache_size = 0: window + exact squared kernel over the evicted tokens
    o = K.hybrid_prefill(dev(q), dev(k), dev(v), window=32, cache_size=0, refresh=16,
                         softmax_scale=scale)
    ref = O.hybrid_prefill(q[0, 0], k[0, 0], v[0, 0], 32, 0, 16, scale)["o"]
    assert_close(host(o)[0, 0], ref, RTOL_F32, "empty cache")


def test_hybrid_2x16x16384_full_size(K):
    cfg = S.CONFIGS["hybrid_2x16x16384"]
    c = S.hybrid_case("full", cfg["B"], cfg["H"], cfg["T"], cfg["d"], cfg["window"],
                      cfg["cache_size"], cfg["refresh"], cfg["seed"], threads=16)
    heads = [(0, 0), (0, 5), (0, 10), (0, 15), (1, 0), (1, 6), (1, 11), (1, 15)]
    _hybrid_check(K, c, heads, torch.bfloat16, RTOL_BF16, aux=True)
