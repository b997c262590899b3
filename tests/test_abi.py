"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol the header declares, and rejects bad arguments on the host (with a
status code and a message) before anything would be enqueued. Pointers here
are dummies that the library never dereferences on these paths."""
import ctypes
import os
import re

import pytest

from kernelized_linear_attention_02_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p(0x10000)  # dummy device pointer, never dereferenced here


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_exports_match_header(lib):
    hdr = open(os.path.join(ROOT, "include", "kla.h")).read()
    declared = set(re.findall(r"KLA_API\s+[\w\s\*]+?\b(kla_\w+)\s*\(", hdr))
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.kla_abi_version() == int(re.search(r"#define KLA_ABI_VERSION (\d+)", hdr).group(1))


def test_small_helpers(lib):
    assert lib.kla_phi_dim(64) == 2080 and lib.kla_phi_dim(16) == 136 and lib.kla_phi_dim(0) == -1
    assert lib.kla_status_string(0) == b"ok"
    assert lib.kla_status_string(3) == b"workspace too small"


def _shape(**kw):
    d = dict(B=1, H=2, T=100, d_qk=64, d_v=64, in_dtype=B.KLA_BF16, out_dtype=B.KLA_BF16, eps=0.0)
    d.update(kw)
    return B.Shape(**d)


def _prefill(lib, shp, chunk=64, q=P, k=P, v=P, o=P, H0=None, s0=None, HT=None, sT=None, ws=P,
             nbytes=1 << 40):
    return lib.kla_prefill(ctypes.byref(shp) if shp is not None else None, chunk, q, k, v, o, H0, s0,
                           HT, sT, ws, nbytes, None)


@pytest.mark.parametrize("kw,chunk,status", [
    (dict(T=0), 64, B.KLA_ERR_INVALID_ARGUMENT),
    (dict(B=0), 64, B.KLA_ERR_INVALID_ARGUMENT),
    (dict(d_qk=48), 64, B.KLA_ERR_UNSUPPORTED),
    (dict(d_v=8), 64, B.KLA_ERR_UNSUPPORTED),
    (dict(in_dtype=7), 64, B.KLA_ERR_UNSUPPORTED),
    (dict(eps=-1.0), 64, B.KLA_ERR_INVALID_ARGUMENT),
    (dict(eps=float("nan")), 64, B.KLA_ERR_INVALID_ARGUMENT),
    (dict(), 48, B.KLA_ERR_UNSUPPORTED),
    (dict(B=300, H=300), 64, B.KLA_ERR_UNSUPPORTED),
])
def test_prefill_rejects_bad_shapes(lib, kw, chunk, status):
    assert _prefill(lib, _shape(**kw), chunk) == status
    assert lib.kla_last_error() != b""


def test_prefill_rejects_bad_pointers(lib):
    shp = _shape()
    assert _prefill(lib, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert _prefill(lib, shp, q=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert _prefill(lib, shp, H0=P) == B.KLA_ERR_INVALID_ARGUMENT  # s0 missing
    assert _prefill(lib, shp, HT=P) == B.KLA_ERR_INVALID_ARGUMENT  # s_T missing
    assert _prefill(lib, shp, o=None) == B.KLA_ERR_INVALID_ARGUMENT  # no output at all
    assert b"o may be NULL" in lib.kla_last_error()


def test_prefill_workspace_checks(lib):
    shp = _shape()
    need = ctypes.c_size_t(0)
    assert lib.kla_prefill_workspace_size(ctypes.byref(shp), 64, 1, ctypes.byref(need)) == B.KLA_OK
    assert need.value > 0
    assert _prefill(lib, shp, ws=None) == B.KLA_ERR_WORKSPACE
    assert _prefill(lib, shp, nbytes=need.value - 1) == B.KLA_ERR_WORKSPACE
    # state-only mode needs no output partials
    none = ctypes.c_size_t(123)
    assert lib.kla_prefill_workspace_size(ctypes.byref(shp), 64, 0, ctypes.byref(none)) == B.KLA_OK
    assert none.value <= need.value
    assert lib.kla_prefill_workspace_size(ctypes.byref(shp), 64, 1, None) == B.KLA_ERR_INVALID_ARGUMENT


def _sre(n_cand=64, top_k=16, ck=P, cv=P, sel=P, sk=None, sv=None):
    return B.SreArgs(n_cand, top_k, ck.value if ck else None, cv.value if cv else None, None,
                     sel.value if sel else None, sk.value if sk else None, sv.value if sv else None)


def _decode(lib, N=8, dqk=64, dv=64, sre=None, H=P, o=P, ws=P, nbytes=1 << 40, eps=0.0):
    return lib.kla_decode_step(N, dqk, dv, eps, H, P, P, P, P, B.KLA_F32, o, B.KLA_F32,
                               ctypes.byref(sre) if sre is not None else None, ws, nbytes, None)


def test_decode_and_sre_validation(lib):
    assert _decode(lib, N=0) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, dqk=24) == B.KLA_ERR_UNSUPPORTED
    assert _decode(lib, H=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, o=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, eps=float("inf")) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, sre=_sre(top_k=65)) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, sre=_sre(top_k=0)) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, sre=_sre(n_cand=300, top_k=4)) == B.KLA_ERR_UNSUPPORTED
    assert _decode(lib, sre=_sre(sel=None)) == B.KLA_ERR_INVALID_ARGUMENT
    assert _decode(lib, sre=_sre(sk=P)) == B.KLA_ERR_INVALID_ARGUMENT  # sel_v missing
    # gathered outputs must not overlap the candidates
    ck = ctypes.c_void_p(0x100000)
    cv = ctypes.c_void_p(0x900000)
    bad = _sre(ck=ck, cv=cv, sk=ctypes.c_void_p(0x100000 + 64), sv=ctypes.c_void_p(0x2000000))
    assert _decode(lib, N=1, sre=bad) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"overlap" in lib.kla_last_error()
    # no scores pointer: the vector-unit scorer (d = 32) keeps them in the workspace
    need = ctypes.c_size_t(0)
    s = _sre()
    assert lib.kla_decode_workspace_size(8, 32, 32, ctypes.byref(s), ctypes.byref(need)) == B.KLA_OK
    assert need.value >= 8 * 64 * 4
    assert _decode(lib, dqk=32, dv=32, sre=_sre(), ws=None) == B.KLA_ERR_WORKSPACE
    # the fused matrix-core step (d = 64, at most 64 candidates) needs none
    assert lib.kla_decode_workspace_size(8, 64, 64, ctypes.byref(s), ctypes.byref(need)) == B.KLA_OK
    assert need.value == 0
    s65 = _sre(n_cand=65)
    assert lib.kla_decode_workspace_size(8, 64, 64, ctypes.byref(s65), ctypes.byref(need)) == B.KLA_OK
    assert need.value >= 8 * 65 * 4
    assert lib.kla_sre_select(8, 64, 64, 0.0, None, P, ctypes.byref(s), P, 1 << 40, None) == \
        B.KLA_ERR_INVALID_ARGUMENT
    assert lib.kla_sre_select(8, 64, 64, 0.0, P, P, None, P, 1 << 40, None) == B.KLA_ERR_INVALID_ARGUMENT


def test_decode_deferred_validation(lib):
    Hp, sp, pk, pv = (ctypes.c_void_p(x) for x in (0x10000000, 0x20000000, 0x30000000, 0x40000000))
    Pn = lib.kla_decode_pending_period()
    assert Pn == 8

    def step(N=8, d=64, H=Hp, s=sp, k=pk, v=pv, n_pend=0, sre=None):
        return lib.kla_decode_step_deferred(N, d, d, 0.0, H, s, k, v, n_pend, P, P, P, B.KLA_F32, P, B.KLA_F32,
                                            ctypes.byref(sre) if sre is not None else None, None)
    assert step(n_pend=-1) == B.KLA_ERR_INVALID_ARGUMENT
    assert step(n_pend=Pn) == B.KLA_ERR_INVALID_ARGUMENT
    assert step(k=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert step(v=pk) == B.KLA_ERR_INVALID_ARGUMENT                   # pend_k and pend_v overlap
    assert step(k=ctypes.c_void_p(0x10000000 + 4096)) == B.KLA_ERR_INVALID_ARGUMENT  # pend_k inside H
    assert step(k=ctypes.c_void_p(0x30000004)) == B.KLA_ERR_INVALID_ARGUMENT         # misaligned
    assert step(d=32) == B.KLA_ERR_UNSUPPORTED
    assert step(sre=_sre(n_cand=65, top_k=16)) == B.KLA_ERR_UNSUPPORTED
    assert step(sre=_sre(n_cand=16, top_k=17)) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"n_pend" in lib.kla_last_error() or True
    fl = lib.kla_decode_flush
    assert fl(8, 64, 64, Hp, sp, pk, pv, Pn, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert fl(8, 64, 64, Hp, sp, pk, pk, 1, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert fl(8, 64, 64, None, sp, pk, pv, 1, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert fl(8, 16, 16, Hp, sp, pk, pv, 1, None) == B.KLA_ERR_UNSUPPORTED


def test_hybrid_validation(lib):
    shp = _shape(T=1000)

    def call(cfg, o=P, ws=P, nbytes=1 << 40, HT=None, sT=None):
        return lib.kla_hybrid_prefill(ctypes.byref(shp), ctypes.byref(cfg) if cfg else None, P, P, P,
                                      o, HT, sT, None, None, ws, nbytes, None)

    assert call(None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(B.HybridCfg(512, 128, 0, 0.125)) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(B.HybridCfg(-1, 128, 64, 0.125)) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(B.HybridCfg(512, 200, 64, 0.125)) == B.KLA_ERR_UNSUPPORTED
    assert call(B.HybridCfg(512, 128, 200, 0.125)) == B.KLA_ERR_UNSUPPORTED
    assert call(B.HybridCfg(512, 128, 64, float("inf"))) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(B.HybridCfg(512, 128, 64, 0.125), o=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(B.HybridCfg(512, 128, 64, 0.125), HT=P) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(B.HybridCfg(512, 128, 64, 0.125), ws=None) == B.KLA_ERR_WORKSPACE
    need = ctypes.c_size_t(0)
    cfg = B.HybridCfg(512, 128, 64, 0.125)
    assert lib.kla_hybrid_workspace_size(ctypes.byref(shp), ctypes.byref(cfg), ctypes.byref(need)) == B.KLA_OK
    assert call(cfg, nbytes=need.value - 1) == B.KLA_ERR_WORKSPACE


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    import kernelized_linear_attention_02_amd as K
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        K.prefill(x, x, x, chunk=32)


def test_prefill_quadratic_rejects(lib):
    call = lib.kla_prefill_quadratic
    assert call(None, P, P, P, P, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(_shape()), None, P, P, P, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(_shape()), P, P, P, None, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"required" in lib.kla_last_error()
    # only d = 64 with bf16 inputs
    assert call(ctypes.byref(_shape(d_qk=32, d_v=32)), P, P, P, P, None, None) == B.KLA_ERR_UNSUPPORTED
    assert call(ctypes.byref(_shape(in_dtype=B.KLA_F32)), P, P, P, P, None, None) == B.KLA_ERR_UNSUPPORTED
    assert call(ctypes.byref(_shape(eps=-1.0)), P, P, P, P, None, None) == B.KLA_ERR_INVALID_ARGUMENT


def test_prefill_quadratic_factors_rejects(lib):
    call = lib.kla_prefill_quadratic_factors
    shp = ctypes.byref(_shape())
    assert call(None, 0, 2, P, P, P, P, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(shp, 0, 2, P, P, P, None, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(shp, 2, 2, P, P, P, P, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"kind" in lib.kla_last_error()
    for g in (0, 3, 8, -1):
        assert call(shp, B.KLA_FACTORS_SUM, g, P, P, P, P, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"factors" in lib.kla_last_error()
    assert call(ctypes.byref(_shape(d_qk=32, d_v=32)), 0, 2, P, P, P, P, None, None) == B.KLA_ERR_UNSUPPORTED
    assert call(ctypes.byref(_shape(in_dtype=B.KLA_F32)), 1, 4, P, P, P, P, None, None) == B.KLA_ERR_UNSUPPORTED


def test_prefill_factors_workspace_query(lib):
    q = lib.kla_prefill_factors_workspace_size
    shp = ctypes.byref(_shape())
    n = ctypes.c_size_t(0)
    assert q(shp, 64, B.KLA_FACTORS_SUM, 2, 1, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert q(None, 64, B.KLA_FACTORS_SUM, 2, 1, ctypes.byref(n)) == B.KLA_ERR_INVALID_ARGUMENT
    assert q(shp, 48, B.KLA_FACTORS_SUM, 2, 1, ctypes.byref(n)) == B.KLA_ERR_UNSUPPORTED
    assert q(shp, 64, 7, 2, 1, ctypes.byref(n)) == B.KLA_ERR_INVALID_ARGUMENT
    assert q(shp, 64, B.KLA_FACTORS_SUM, 3, 1, ctypes.byref(n)) == B.KLA_ERR_INVALID_ARGUMENT
    sizes = {}
    for kind in (B.KLA_FACTORS_CONCAT, B.KLA_FACTORS_SUM):
        for g in (1, 2, 4):
            assert q(shp, 64, kind, g, 1, ctypes.byref(n)) == B.KLA_OK
            sizes[kind, g] = n.value
    # one factor is kla_prefill for either kind
    base = ctypes.c_size_t(0)
    assert lib.kla_prefill_workspace_size(shp, 64, 1, ctypes.byref(base)) == B.KLA_OK
    assert sizes[B.KLA_FACTORS_CONCAT, 1] == sizes[B.KLA_FACTORS_SUM, 1] == base.value
    # the concatenated lift fits kla_prefill's workspace, as documented
    assert sizes[B.KLA_FACTORS_CONCAT, 2] <= base.value and sizes[B.KLA_FACTORS_CONCAT, 4] <= base.value
    assert sizes[B.KLA_FACTORS_SUM, 2] > 0


def test_prefill_factors_rejects(lib):
    call = lib.kla_prefill_factors
    shp = ctypes.byref(_shape())

    def go(kind=B.KLA_FACTORS_CONCAT, g=2, shape=shp, chunk=64):
        return call(shape, chunk, kind, g, P, P, P, P, None, None, None, None, P, 1 << 40, None)
    assert go(kind=5) == B.KLA_ERR_INVALID_ARGUMENT
    # the summed lift is served (vector path): with a huge workspace claim the
    # checks pass up to the launch, which has no GPU here
    for g in (0, 3, 8):
        assert go(kind=B.KLA_FACTORS_SUM, g=g) == B.KLA_ERR_INVALID_ARGUMENT
    for g in (0, 3, 8):
        assert go(g=g) == B.KLA_ERR_INVALID_ARGUMENT
    assert go(chunk=48) == B.KLA_ERR_UNSUPPORTED
    assert go(shape=ctypes.byref(_shape(d_qk=48, d_v=32))) == B.KLA_ERR_UNSUPPORTED
    assert go(shape=None) == B.KLA_ERR_INVALID_ARGUMENT


def test_prefill_quadratic_backward_rejects(lib):
    call = lib.kla_prefill_quadratic_backward
    shp = ctypes.byref(_shape())

    def go(shape=shp, den=P, ws=P, nbytes=1 << 40, dq=P):
        return call(shape, P, P, P, den, P, dq, P, P, ws, nbytes, None)

    assert go(shape=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert go(den=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert go(dq=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"required" in lib.kla_last_error()
    assert go(shape=ctypes.byref(_shape(d_qk=32, d_v=32))) == B.KLA_ERR_UNSUPPORTED
    assert go(shape=ctypes.byref(_shape(in_dtype=B.KLA_F32))) == B.KLA_ERR_UNSUPPORTED
    need = ctypes.c_size_t(0)
    assert lib.kla_prefill_quadratic_backward_workspace_size(shp, ctypes.byref(need)) == B.KLA_OK
    assert need.value >= 2 * 100 * 4  # c for B*H*T tokens
    assert go(ws=None) == B.KLA_ERR_WORKSPACE
    assert go(nbytes=need.value - 1) == B.KLA_ERR_WORKSPACE
    assert lib.kla_prefill_quadratic_backward_workspace_size(None, ctypes.byref(need)) == \
        B.KLA_ERR_INVALID_ARGUMENT


def _hstate(*ptrs, row=B.KLA_BF16):
    """A hybrid decode state of fake device pointers whose rows are bf16 (the
    in_dtype these checks pass)."""
    return B.HybridState(*ptrs, row)


def test_hybrid_decode_validation(lib):
    st = _hstate(*([0x10000] * 10))
    cfg = B.HybridCfg(512, 128, 1, 0.125)

    def call(cfg=cfg, N=8, dqk=64, dv=64, t=600, state=st, o=P, ws=P, nbytes=1 << 40, eps=0.0,
             in_dtype=B.KLA_BF16):
        return lib.kla_hybrid_decode_step(N, dqk, dv, eps, ctypes.byref(cfg) if cfg else None, t,
                                          ctypes.byref(state) if state else None, P, P, P, in_dtype, o,
                                          B.KLA_F32, None, ws, nbytes, None)

    assert call(cfg=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(N=0) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(dqk=48) == B.KLA_ERR_UNSUPPORTED
    assert call(cfg=B.HybridCfg(512, 128, 64, 0.125)) == B.KLA_ERR_UNSUPPORTED
    assert b"refresh = 1" in lib.kla_last_error()
    assert call(cfg=B.HybridCfg(-1, 128, 1, 0.125)) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(cfg=B.HybridCfg(512, 256, 1, 0.125)) == B.KLA_ERR_UNSUPPORTED
    assert call(cfg=B.HybridCfg(512, 128, 1, float("nan"))) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(t=-1) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(eps=-1.0) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(in_dtype=7) == B.KLA_ERR_UNSUPPORTED
    assert call(state=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(o=None) == B.KLA_ERR_INVALID_ARGUMENT
    no_cache = _hstate(0x10000, 0x10000, 0x10000, 0x10000, None, None, None, 0x10000, 0x10000, None)
    assert call(state=no_cache) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"cache_size > 0" in lib.kla_last_error()
    # without a cache, the cache pointers may be NULL (only the workspace check is left)
    assert call(cfg=B.HybridCfg(512, 0, 1, 0.125), state=no_cache, ws=None) == B.KLA_ERR_WORKSPACE
    odd = _hstate(0x10000, 0x10004, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
    assert call(state=odd) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.kla_last_error()
    odd_sums = _hstate(*([0x10000] * 9), 0x10004)
    assert call(state=odd_sums) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.kla_last_error()
    no_sums = _hstate(*([0x10000] * 9), None)
    assert call(state=no_sums) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"cache_sums" in lib.kla_last_error()
    no_pend = _hstate(*([0x10000] * 7), None, None, 0x10000)
    assert call(state=no_pend) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"pend_k" in lib.kla_last_error()
    # the window and cache rows must be in the step's input type
    f32_rows = _hstate(*([0x10000] * 10), row=B.KLA_F32)
    assert call(state=f32_rows) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"row_dtype" in lib.kla_last_error()

    need = ctypes.c_size_t(0)
    assert lib.kla_hybrid_decode_workspace_size(8, 64, 64, ctypes.byref(cfg), ctypes.byref(need)) == B.KLA_OK
    assert need.value >= 2 * 8 * 65 * 4  # linear readouts of q and of the evicted key
    assert call(ws=None) == B.KLA_ERR_WORKSPACE
    assert call(nbytes=need.value - 1) == B.KLA_ERR_WORKSPACE
    assert lib.kla_hybrid_decode_workspace_size(8, 64, 64, None, ctypes.byref(need)) == \
        B.KLA_ERR_INVALID_ARGUMENT

    flush = lib.kla_hybrid_decode_flush
    assert flush(8, 64, 64, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    assert flush(8, 64, 64, ctypes.byref(no_pend), None) == B.KLA_ERR_INVALID_ARGUMENT
    assert flush(0, 64, 64, ctypes.byref(st), None) == B.KLA_ERR_INVALID_ARGUMENT
    assert flush(8, 48, 64, ctypes.byref(st), None) == B.KLA_ERR_UNSUPPORTED

    prime = lib.kla_hybrid_decode_prime
    assert prime(8, 64, 64, ctypes.byref(cfg), 600, None, None) == B.KLA_ERR_INVALID_ARGUMENT
    bad_rows = _hstate(*([0x10000] * 10), row=7)
    assert prime(8, 64, 64, ctypes.byref(cfg), 600, ctypes.byref(bad_rows), None) == B.KLA_ERR_UNSUPPORTED
    assert prime(8, 64, 64, None, 600, ctypes.byref(st), None) == B.KLA_ERR_INVALID_ARGUMENT
    assert prime(8, 64, 64, ctypes.byref(cfg), -1, ctypes.byref(st), None) == B.KLA_ERR_INVALID_ARGUMENT
    assert prime(8, 48, 64, ctypes.byref(cfg), 600, ctypes.byref(st), None) == B.KLA_ERR_UNSUPPORTED
    assert prime(8, 64, 64, ctypes.byref(cfg), 600, ctypes.byref(no_sums), None) == B.KLA_ERR_INVALID_ARGUMENT
    assert prime(8, 64, 64, ctypes.byref(cfg), 600, ctypes.byref(odd_sums), None) == B.KLA_ERR_INVALID_ARGUMENT


M = ctypes.c_void_p(0x10008)  # 8-byte aligned only: every call must refuse it


def test_hybrid_decode_static_validation(lib):
    # host-side checks of the allocation-free step: the same argument checks
    # as the workspace step, then the static scratch limit (all before any
    # device call, so they run without a GPU)
    assert lib.kla_hybrid_decode_static_limit() == 16 << 20
    # the pending slots of a hybrid decode state, as the header declares them
    hdr = open(os.path.join(ROOT, "include", "kla.h")).read()
    assert lib.kla_hybrid_decode_pending_slots() == int(re.search(r"#define KLA_HYBRID_PENDING (\d+)", hdr).group(1))
    st = _hstate(*([0x10000] * 10))
    cfg = B.HybridCfg(512, 128, 1, 0.125)

    def call(cfg=cfg, N=8, t=600, state=st, o=P, q=P):
        return lib.kla_hybrid_decode_step_static(N, 64, 64, 0.0, ctypes.byref(cfg) if cfg else None, t,
                                                 ctypes.byref(state) if state else None, q, P, P, B.KLA_BF16,
                                                 o, B.KLA_F32, None, None)

    assert call(cfg=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(N=0) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(t=-1) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(state=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(o=None) == B.KLA_ERR_INVALID_ARGUMENT
    assert call(q=ctypes.c_void_p(0x10004)) == B.KLA_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.kla_last_error()
    # two readouts of 68 floats per head-state: 30800 fit in 16 MiB
    need = ctypes.c_size_t(0)
    assert lib.kla_hybrid_decode_workspace_size(30800, 64, 64, ctypes.byref(cfg), ctypes.byref(need)) == 0
    assert need.value <= 16 << 20
    assert lib.kla_hybrid_decode_workspace_size(31000, 64, 64, ctypes.byref(cfg), ctypes.byref(need)) == 0
    assert need.value > 16 << 20
    assert call(N=31000) == B.KLA_ERR_UNSUPPORTED
    assert b"static" in lib.kla_last_error()


def _misaligned(lib, status):
    assert status == B.KLA_ERR_INVALID_ARGUMENT
    assert b"16-byte aligned" in lib.kla_last_error()


def test_every_call_rejects_misaligned_pointers(lib):
    shp = _shape()
    # prefill: each device pointer in turn
    for kw in ("q", "k", "v", "o", "ws"):
        _misaligned(lib, _prefill(lib, shp, **{kw: M}))
    _misaligned(lib, _prefill(lib, shp, H0=M, s0=P))
    _misaligned(lib, _prefill(lib, shp, HT=P, sT=M))
    _misaligned(lib, lib.kla_prefill_factors(ctypes.byref(shp), 64, 0, 2, P, M, P, P, None, None, None, None, P,
                                             1 << 40, None))
    # quadratic form and its backward
    _misaligned(lib, lib.kla_prefill_quadratic(ctypes.byref(shp), P, P, M, P, None, None))
    _misaligned(lib, lib.kla_prefill_quadratic(ctypes.byref(shp), P, P, P, P, M, None))
    _misaligned(lib, lib.kla_prefill_quadratic_factors(ctypes.byref(shp), 1, 2, M, P, P, P, None, None))
    _misaligned(lib, lib.kla_prefill_quadratic_backward(ctypes.byref(shp), P, P, P, P, M, P, P, P, P, 1 << 40,
                                                        None))
    # decode, with and without selection; scoring alone
    _misaligned(lib, _decode(lib, H=M))
    _misaligned(lib, _decode(lib, o=M))
    _misaligned(lib, _decode(lib, sre=_sre(ck=M)))
    _misaligned(lib, _decode(lib, sre=_sre(sel=M)))
    s = _sre()
    _misaligned(lib, lib.kla_sre_select(8, 64, 64, 0.0, M, P, ctypes.byref(s), P, 1 << 40, None))
    _misaligned(lib, lib.kla_sre_select(8, 64, 64, 0.0, P, P, ctypes.byref(_sre(cv=M)), P, 1 << 40, None))
    # hybrid prefill (both entry points)
    cfg = B.HybridCfg(512, 128, 64, 0.125)
    _misaligned(lib, lib.kla_hybrid_prefill(ctypes.byref(shp), ctypes.byref(cfg), P, M, P, P, None, None, None,
                                            None, P, 1 << 40, None))
    _misaligned(lib, lib.kla_hybrid_prefill_streams(ctypes.byref(shp), ctypes.byref(cfg), P, P, P, P, None, None,
                                                    None, M, P, 1 << 40, None, None))
    # token-by-token hybrid decode, its flush and its prime
    st = _hstate(*([0x10000] * 10))
    hcfg = B.HybridCfg(512, 128, 1, 0.125)
    _misaligned(lib, lib.kla_hybrid_decode_step(8, 64, 64, 0.0, ctypes.byref(hcfg), 600, ctypes.byref(st), P, P,
                                                M, B.KLA_BF16, P, B.KLA_F32, None, P, 1 << 40, None))
    bad_pend = _hstate(*([0x10000] * 7), 0x10004, 0x10000, 0x10000)
    _misaligned(lib, lib.kla_hybrid_decode_flush(8, 64, 64, ctypes.byref(bad_pend), None))
    _misaligned(lib, lib.kla_hybrid_decode_prime(8, 64, 64, ctypes.byref(hcfg), 600, ctypes.byref(bad_pend), None))


def test_hybrid_streams_entry_validates_like_the_plain_one(lib):
    shp = _shape(T=1000)
    cfg = B.HybridCfg(512, 200, 64, 0.125)
    assert lib.kla_hybrid_prefill_streams(ctypes.byref(shp), ctypes.byref(cfg), P, P, P, P, None, None, None,
                                          None, P, 1 << 40, None, None) == B.KLA_ERR_UNSUPPORTED
    cfg = B.HybridCfg(512, 128, 64, 0.125)
    assert lib.kla_hybrid_prefill_streams(ctypes.byref(shp), ctypes.byref(cfg), P, P, P, None, None, None, None,
                                          None, P, 1 << 40, None, None) == B.KLA_ERR_INVALID_ARGUMENT


def test_binding_copies_misaligned_views():
    torch = pytest.importorskip("torch")
    from kernelized_linear_attention_02_amd._binding import _dense
    x = torch.arange(40, dtype=torch.float32)[1:33]  # storage offset of 4 bytes
    assert x.data_ptr() % 16 != 0
    y = _dense(x)
    assert y.data_ptr() % 16 == 0 and torch.equal(x, y)
