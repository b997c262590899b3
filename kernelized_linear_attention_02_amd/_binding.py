"""ctypes binding of libkla's C ABI (include/kla.h).

Argument marshalling only: these functions check Python-level types,
allocate outputs and workspace with ``torch.empty`` on the inputs' device,
and pass raw device pointers and the current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is
no fallback. If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkla.so")

KLA_OK, KLA_ERR_INVALID_ARGUMENT, KLA_ERR_UNSUPPORTED, KLA_ERR_WORKSPACE, KLA_ERR_HIP = range(5)
KLA_F32, KLA_BF16 = 0, 1
KLA_FACTORS_CONCAT, KLA_FACTORS_SUM = 0, 1

EXPORTS = (
    "kla_abi_version", "kla_phi_dim", "kla_status_string", "kla_last_error",
    "kla_prefill_matrix_path", "kla_prefill_workspace_size", "kla_prefill", "kla_prefill_quadratic",
    "kla_prefill_quadratic_factors", "kla_prefill_factors", "kla_prefill_factors_workspace_size", "kla_prefill_quadratic_backward_workspace_size", "kla_prefill_quadratic_backward",
    "kla_decode_workspace_size", "kla_decode_step",
    "kla_decode_pending_period", "kla_decode_step_deferred", "kla_decode_flush",
    "kla_sre_workspace_size", "kla_sre_select",
    "kla_hybrid_workspace_size", "kla_hybrid_prefill", "kla_hybrid_prefill_streams",
    "kla_hybrid_decode_workspace_size", "kla_hybrid_decode_step", "kla_hybrid_decode_flush",
    "kla_hybrid_decode_prime", "kla_hybrid_decode_static_limit", "kla_hybrid_decode_step_static",
    "kla_hybrid_decode_pending_slots",
    "kla_profile_enable", "kla_profile_read",
)


class KlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
                ("d_qk", ctypes.c_int), ("d_v", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("eps", ctypes.c_float)]


class SreArgs(ctypes.Structure):
    _fields_ = [("n_cand", ctypes.c_int), ("top_k", ctypes.c_int),
                ("cand_k", ctypes.c_void_p), ("cand_v", ctypes.c_void_p),
                ("scores", ctypes.c_void_p), ("sel", ctypes.c_void_p),
                ("sel_k", ctypes.c_void_p), ("sel_v", ctypes.c_void_p),
                ("sel_stride", ctypes.c_int)]


class HybridCfg(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int), ("cache_size", ctypes.c_int),
                ("refresh", ctypes.c_int), ("softmax_scale", ctypes.c_float)]


class HybridState(ctypes.Structure):
    _fields_ = [("H", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("win_k", ctypes.c_void_p), ("win_v", ctypes.c_void_p),
                ("cache_k", ctypes.c_void_p), ("cache_v", ctypes.c_void_p),
                ("cache_ids", ctypes.c_void_p), ("pend_k", ctypes.c_void_p), ("pend_v", ctypes.c_void_p),
                ("cache_sums", ctypes.c_void_p), ("row_dtype", ctypes.c_int)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkla.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkla.so not found at {path}; build it with "
                          f"`python -m kernelized_linear_attention_02_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    szp = ctypes.POINTER(ctypes.c_size_t)
    shp = ctypes.POINTER(Shape)
    srp = ctypes.POINTER(SreArgs)
    hcp = ctypes.POINTER(HybridCfg)
    hsp = ctypes.POINTER(HybridState)
    sig = {
        "kla_abi_version": (i, []),
        "kla_phi_dim": (i, [i]),
        "kla_status_string": (ctypes.c_char_p, [i]),
        "kla_last_error": (ctypes.c_char_p, []),
        "kla_prefill_matrix_path": (i, [shp, i]),
        "kla_prefill_workspace_size": (i, [shp, i, i, szp]),
        "kla_prefill": (i, [shp, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "kla_prefill_quadratic": (i, [shp, vp, vp, vp, vp, vp, vp]),
        "kla_prefill_quadratic_factors": (i, [shp, i, i, vp, vp, vp, vp, vp, vp]),
        "kla_prefill_factors": (i, [shp, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "kla_prefill_factors_workspace_size": (i, [shp, i, i, i, i, szp]),
        "kla_prefill_quadratic_backward_workspace_size": (i, [shp, szp]),
        "kla_prefill_quadratic_backward": (i, [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "kla_decode_workspace_size": (i, [i, i, i, srp, szp]),
        "kla_decode_step": (i, [i, i, i, f, vp, vp, vp, vp, vp, i, vp, i, srp, vp, sz, vp]),
        "kla_decode_pending_period": (i, []),
        "kla_decode_step_deferred": (i, [i, i, i, f, vp, vp, vp, vp, i, vp, vp, vp, i, vp, i, srp, vp]),
        "kla_decode_flush": (i, [i, i, i, vp, vp, vp, vp, i, vp]),
        "kla_sre_workspace_size": (i, [i, i, i, srp, szp]),
        "kla_sre_select": (i, [i, i, i, f, vp, vp, srp, vp, sz, vp]),
        "kla_hybrid_workspace_size": (i, [shp, hcp, szp]),
        "kla_hybrid_prefill": (i, [shp, hcp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "kla_hybrid_prefill_streams": (i, [shp, hcp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]),
        "kla_hybrid_decode_workspace_size": (i, [i, i, i, hcp, szp]),
        "kla_hybrid_decode_step": (i, [i, i, i, f, hcp, i, hsp, vp, vp, vp, i, vp, i, vp, vp, sz, vp]),
        "kla_hybrid_decode_flush": (i, [i, i, i, hsp, vp]),
        "kla_hybrid_decode_prime": (i, [i, i, i, hcp, i, hsp, vp]),
        "kla_hybrid_decode_static_limit": (sz, []),
        "kla_hybrid_decode_pending_slots": (i, []),
        "kla_hybrid_decode_step_static": (i, [i, i, i, f, hcp, i, hsp, vp, vp, vp, i, vp, i, vp, vp]),
        "kla_profile_enable": (i, [i]),
        "kla_profile_read": (i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int),
                                 ctypes.POINTER(ctypes.c_int)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int):
    if status != KLA_OK:
        lib = load_library()
        raise KlaError(status, lib.kla_last_error().decode())


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return KLA_F32
    if t.dtype == torch.bfloat16:
        return KLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _torch_dtype(code: int):
    torch = _torch()
    return torch.float32 if code == KLA_F32 else torch.bfloat16


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dense(t):
    """A contiguous tensor whose data pointer is 16-byte aligned (the library
    rejects misaligned pointers): views at an odd storage offset are copied
    into fresh storage. Values are unchanged."""
    t = t.contiguous()
    if t.data_ptr() % 16:
        t = t.clone()
    return t


def _need_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libkla works on device tensors only")


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


def phi_dim(d: int) -> int:
    return load_library().kla_phi_dim(int(d))


def prefill_uses_matrix_cores(B=4, H=8, T=4096, d_qk=64, d_v=64, chunk=64, dtype=KLA_BF16) -> bool:
    """Whether kla_prefill runs the bf16 matrix-core kernel for this shape."""
    shp = Shape(B, H, T, d_qk, d_v, dtype, dtype, 0.0)
    return load_library().kla_prefill_matrix_path(ctypes.byref(shp), int(chunk)) == 1


def prefill(q, k, v, chunk: int = 64, state=None, return_state: bool = False, eps: float = 0.0,
            out_dtype=None, outputs: bool = True, out=None, factors: int = 1, factor_kind: str = "concat"):
    """Chunked causal prefill. q, k [B, H, T, d_qk]; v [B, H, T, d_v] (float32 or
    bfloat16, same dtype). ``state`` = (H0, s0) float32 resumes a previous call.
    Returns o, or (o, H_T, s_T) with ``return_state``; with ``outputs=False``
    only (H_T, s_T). ``factors`` > 1 selects a multi-factor lift
    (kla_prefill_factors; any supported shape): ``factor_kind`` "concat"
    (KATA-Mg) or "sum" (KATA-Sigma-g), whose state has
    factor_phi_dim(d_qk, factors, factor_kind) features."""
    torch = _torch()
    lib = load_library()
    _need_device(q, k, v)
    q, k, v = _dense(q), _dense(k), _dense(v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hh, T, dqk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch between q, k and v")
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    shp = Shape(B, Hh, T, dqk, dv, code, ocode, float(eps))
    if factor_kind not in FACTOR_KINDS:
        raise ValueError(f"factor_kind must be one of {tuple(FACTOR_KINDS)}")
    D = phi_dim(dqk) if factors == 1 else factor_phi_dim(dqk, factors, factor_kind)
    dev = q.device
    if outputs and out is not None:
        if out.shape != (B, Hh, T, dv) or out.dtype != _torch_dtype(ocode) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B, H, T, d_v] tensor of the output dtype")
        o = out
    else:
        o = torch.empty((B, Hh, T, dv), dtype=_torch_dtype(ocode), device=dev) if outputs else None
    want_state = return_state or not outputs
    HT = torch.empty((B, Hh, D, dv), dtype=torch.float32, device=dev) if want_state else None
    sT = torch.empty((B, Hh, D), dtype=torch.float32, device=dev) if want_state else None
    H0 = s0 = None
    if state is not None:
        H0, s0 = (_dense(x) for x in state)
        _need_device(H0, s0)
        if H0.dtype != torch.float32 or s0.dtype != torch.float32:
            raise TypeError("state must be float32")
        if H0.numel() != B * Hh * D * dv or s0.numel() != B * Hh * D:
            raise ValueError("state shape does not match [B, H, D, d_v], [B, H, D]")
    nbytes = ctypes.c_size_t(0)
    if factors == 1:
        check(lib.kla_prefill_workspace_size(ctypes.byref(shp), int(chunk), int(outputs), ctypes.byref(nbytes)))
    else:
        check(lib.kla_prefill_factors_workspace_size(ctypes.byref(shp), int(chunk), FACTOR_KINDS[factor_kind],
                                                     int(factors), int(outputs), ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    if factors == 1:
        check(lib.kla_prefill(ctypes.byref(shp), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                              _ptr(H0), _ptr(s0), _ptr(HT), _ptr(sT), _ptr(ws), nbytes.value,
                              _stream(dev)))
    else:
        check(lib.kla_prefill_factors(ctypes.byref(shp), int(chunk), FACTOR_KINDS[factor_kind], int(factors),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(H0), _ptr(s0), _ptr(HT),
                                      _ptr(sT), _ptr(ws), nbytes.value, _stream(dev)))
    if not outputs:
        return HT, sT
    return (o, HT, sT) if return_state else o


FACTOR_KINDS = {"concat": 0, "sum": 1}


def factor_phi_dim(d: int, factors: int, kind: str = "concat") -> int:
    """State features of a multi-factor lift, p = d / g: g p(p+1)/2 for the
    concatenated lift, p(p+1)/2 for the summed one."""
    p = d // factors
    return (1 if kind == "sum" else factors) * p * (p + 1) // 2


def prefill_quadratic(q, k, v, eps: float = 0.0, out_dtype=None, out=None, return_den: bool = False,
                      factors: int = 1, factor_kind: str = "concat"):
    """Causal prefill in the quadratic form (no state): q, k, v [B, H, T, 64]
    bfloat16. Returns o [B, H, T, 64] (bfloat16, or ``out_dtype``), and with
    ``return_den`` also the row denominators den [B, H, T] float32 (for
    prefill_quadratic_backward). ``factors`` > 1 selects a multi-factor lift
    (kla_prefill_quadratic_factors): ``factor_kind`` "concat" (KATA-Mg,
    weights sum_i (q_i.k_i)^2) or "sum" (KATA-Sigma-g, sum_{i,j} (q_i.k_j)^2)
    over ``factors`` equal slices of the 64 dimensions."""
    torch = _torch()
    lib = load_library()
    _need_device(q, k, v)
    q, k, v = _dense(q), _dense(k), _dense(v)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hh, T, dqk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch between q, k and v")
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    shp = Shape(B, Hh, T, dqk, dv, code, ocode, float(eps))
    if out is not None:
        if out.shape != (B, Hh, T, dv) or out.dtype != _torch_dtype(ocode) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B, H, T, d_v] tensor of the output dtype")
        o = out
    else:
        o = torch.empty((B, Hh, T, dv), dtype=_torch_dtype(ocode), device=q.device)
    den = torch.empty((B, Hh, T), dtype=torch.float32, device=q.device) if return_den else None
    if factors == 1 and factor_kind == "concat":
        check(lib.kla_prefill_quadratic(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                                        _stream(q.device)))
    else:
        if factor_kind not in FACTOR_KINDS:
            raise ValueError(f"factor_kind must be one of {sorted(FACTOR_KINDS)}")
        check(lib.kla_prefill_quadratic_factors(ctypes.byref(shp), FACTOR_KINDS[factor_kind], int(factors),
                                                _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                                                _stream(q.device)))
    return (o, den) if return_den else o


def prefill_quadratic_backward(q, k, v, den, dout, eps: float = 0.0):
    """Gradients (dq, dk, dv) of the causal prefill for dL/do = ``dout``:
    q, k, v [B, H, T, 64] bfloat16; den [B, H, T] float32 from
    prefill_quadratic(..., return_den=True); dout [B, H, T, 64] bfloat16 or
    float32. The gradients come back in the dtype of dout."""
    torch = _torch()
    lib = load_library()
    _need_device(q, k, v, den, dout)
    q, k, v, den, dout = (_dense(x) for x in (q, k, v, den, dout))
    if not (q.dtype == k.dtype == v.dtype) or den.dtype != torch.float32:
        raise TypeError("q, k, v share one dtype; den is float32")
    B, Hh, T, dqk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != q.shape[:3] + (dv,) or dout.shape != v.shape or den.shape != q.shape[:3]:
        raise ValueError("shape mismatch between q, k, v, den and dout")
    shp = Shape(B, Hh, T, dqk, dv, _dtype_code(q), _dtype_code(dout), float(eps))
    dq, dk, dvv = torch.empty_like(dout), torch.empty_like(dout), torch.empty_like(dout)
    nbytes = ctypes.c_size_t(0)
    check(lib.kla_prefill_quadratic_backward_workspace_size(ctypes.byref(shp), ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, q.device)
    check(lib.kla_prefill_quadratic_backward(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(den), _ptr(dout),
                                             _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(ws), nbytes.value,
                                             _stream(q.device)))
    return dq, dk, dvv


def _sre_struct(cand_k, cand_v, top_k, scores, sel, sel_k, sel_v, sel_stride=0):
    return SreArgs(int(cand_k.shape[-2]), int(top_k), cand_k.data_ptr(), cand_v.data_ptr(),
                   None if scores is None else scores.data_ptr(), sel.data_ptr(),
                   None if sel_k is None else sel_k.data_ptr(),
                   None if sel_v is None else sel_v.data_ptr(), int(sel_stride))


def _sre_outputs(N, n_cand, top_k, dqk, dv, device, scores, gather, out=None):
    torch = _torch()
    if out is not None:
        return out["scores"], out["sel"], out.get("sel_k"), out.get("sel_v")
    sc = torch.empty((N, n_cand), dtype=torch.float32, device=device) if scores else None
    sel = torch.empty((N, top_k), dtype=torch.int32, device=device)
    sk = torch.empty((N, top_k, dqk), dtype=torch.float32, device=device) if gather else None
    sv = torch.empty((N, top_k, dv), dtype=torch.float32, device=device) if gather else None
    return sc, sel, sk, sv


def decode_step(H, s, q, k, v, eps: float = 0.0, out_dtype=None, cand_k=None, cand_v=None,
                top_k: int = 0, scores: bool = True, gather: bool = False, out=None):
    """One recurrent token for N head-states; H [N, D, d_v], s [N, D] float32
    updated in place; q, k [N, d_qk], v [N, d_v]. With candidates
    (cand_k [N, n_cand, d_qk], cand_v [N, n_cand, d_v] float32) and top_k,
    also scores and selects against the updated state. ``out`` may pass
    preallocated {'o', 'scores', 'sel', 'sel_k', 'sel_v'} tensors, and
    'sel_stride' when sel_k / sel_v point into a slab with that many rows per
    head (for instance the next step's candidate array).
    Returns o, or (o, dict(scores, sel, sel_k, sel_v))."""
    torch = _torch()
    lib = load_library()
    _need_device(H, s, q, k, v)
    for t in (H, s):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError("H and s must be contiguous float32 (updated in place)")
    q, k, v = _dense(q), _dense(k), _dense(v)
    N, dqk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    dev = q.device
    o = out["o"] if out is not None else torch.empty((N, dv), dtype=_torch_dtype(ocode), device=dev)
    sre_p = None
    res = None
    if cand_k is not None:
        cand_k, cand_v = _dense(cand_k), _dense(cand_v)
        sc, sel, sk, sv = _sre_outputs(N, cand_k.shape[1], top_k, dqk, dv, dev, scores, gather, out)
        stride = 0
        if sk is not None and out is not None and "sel_stride" in out:
            # gathered rows land in a caller slab with `sel_stride` rows per head
            stride = int(out["sel_stride"])
        sre = _sre_struct(cand_k, cand_v, top_k, sc, sel, sk, sv, stride)
        sre_p = ctypes.byref(sre)
        res = dict(scores=sc, sel=sel, sel_k=sk, sel_v=sv)
    nbytes = ctypes.c_size_t(0)
    check(lib.kla_decode_workspace_size(N, dqk, dv, sre_p, ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    check(lib.kla_decode_step(N, dqk, dv, float(eps), _ptr(H), _ptr(s), _ptr(q), _ptr(k), _ptr(v),
                              code, _ptr(o), ocode, sre_p, _ptr(ws), nbytes.value, _stream(dev)))
    return o if res is None else (o, res)


def decode_pending_period() -> int:
    """Tokens per pass that writes the state in decode_step_deferred (P)."""
    return int(load_library().kla_decode_pending_period())


def decode_pending_slots(N: int, d_qk: int = 64, d_v: int = 64, device="cuda"):
    """Zeroed pending slots (pend_k [N, P, d_qk], pend_v [N, P, d_v]) for
    decode_step_deferred."""
    torch = _torch()
    P = decode_pending_period()
    return (torch.zeros((N, P, d_qk), dtype=torch.float32, device=device),
            torch.zeros((N, P, d_v), dtype=torch.float32, device=device))


def decode_step_deferred(H, s, pend_k, pend_v, n_pend: int, q, k, v, eps: float = 0.0, out_dtype=None,
                         cand_k=None, cand_v=None, top_k: int = 0, scores: bool = True, gather: bool = False,
                         out=None):
    """decode_step with deferred folds: the token joins pending slot n_pend
    (H and s only read) until the slots fill, when the call folds all of them
    into H and s. Returns what decode_step returns; the caller's next n_pend
    is (n_pend + 1) % decode_pending_period()."""
    torch = _torch()
    lib = load_library()
    _need_device(H, s, pend_k, pend_v, q, k, v)
    for t in (H, s, pend_k, pend_v):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError("H, s, pend_k and pend_v must be contiguous float32 (updated in place)")
    q, k, v = _dense(q), _dense(k), _dense(v)
    N, dqk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    dev = q.device
    o = out["o"] if out is not None else torch.empty((N, dv), dtype=_torch_dtype(ocode), device=dev)
    sre_p = None
    res = None
    if cand_k is not None:
        cand_k, cand_v = _dense(cand_k), _dense(cand_v)
        sc, sel, sk, sv = _sre_outputs(N, cand_k.shape[1], top_k, dqk, dv, dev, scores, gather, out)
        stride = int(out["sel_stride"]) if (sk is not None and out is not None and "sel_stride" in out) else 0
        sre = _sre_struct(cand_k, cand_v, top_k, sc, sel, sk, sv, stride)
        sre_p = ctypes.byref(sre)
        res = dict(scores=sc, sel=sel, sel_k=sk, sel_v=sv)
    check(lib.kla_decode_step_deferred(N, dqk, dv, float(eps), _ptr(H), _ptr(s), _ptr(pend_k), _ptr(pend_v),
                                       int(n_pend), _ptr(q), _ptr(k), _ptr(v), code, _ptr(o), ocode, sre_p,
                                       _stream(dev)))
    return o if res is None else (o, res)


def decode_flush(H, s, pend_k, pend_v, n_pend: int):
    """Fold the first n_pend pending slots into H and s."""
    lib = load_library()
    _need_device(H, s, pend_k, pend_v)
    N, D, dv = H.shape
    dqk = pend_k.shape[-1]
    check(lib.kla_decode_flush(N, dqk, dv, _ptr(H), _ptr(s), _ptr(pend_k), _ptr(pend_v), int(n_pend),
                               _stream(H.device)))


def sre_select(H, s, cand_k, cand_v, top_k: int, eps: float = 0.0, scores: bool = True,
               gather: bool = False):
    """Score candidates by self-recall error against (H, s) and select the
    top_k. Returns dict(scores, sel, sel_k, sel_v)."""
    torch = _torch()
    lib = load_library()
    _need_device(H, s, cand_k, cand_v)
    H, s = _dense(H), _dense(s)
    cand_k, cand_v = _dense(cand_k), _dense(cand_v)
    if cand_k.dtype != torch.float32 or cand_v.dtype != torch.float32:
        raise TypeError("candidates must be float32")
    N, n_cand, dqk = cand_k.shape
    dv = cand_v.shape[-1]
    dev = cand_k.device
    sc, sel, sk, sv = _sre_outputs(N, n_cand, top_k, dqk, dv, dev, scores, gather)
    sre = _sre_struct(cand_k, cand_v, top_k, sc, sel, sk, sv)
    nbytes = ctypes.c_size_t(0)
    check(lib.kla_sre_workspace_size(N, dqk, dv, ctypes.byref(sre), ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    check(lib.kla_sre_select(N, dqk, dv, float(eps), _ptr(H), _ptr(s), ctypes.byref(sre), _ptr(ws),
                             nbytes.value, _stream(dev)))
    return dict(scores=sc, sel=sel, sel_k=sk, sel_v=sv)


def hybrid_prefill(q, k, v, window: int, cache_size: int, refresh: int, softmax_scale=None,
                   eps: float = 0.0, return_state: bool = False, return_cache: bool = False,
                   return_trace: bool = False, out_dtype=None, aux_stream=None):
    """Window + linear state + sparse cache prefill. Returns o, plus a dict
    with H, s, cache (token ids) and trace when requested. ``aux_stream``
    (a torch.cuda.Stream of the same device, default priority) lets the
    readouts overlap the refresh chain (kla_hybrid_prefill_streams)."""
    torch = _torch()
    lib = load_library()
    _need_device(q, k, v)
    q, k, v = _dense(q), _dense(k), _dense(v)
    B, Hh, T, dqk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    shp = Shape(B, Hh, T, dqk, dv, code, ocode, float(eps))
    cfg = HybridCfg(int(window), int(cache_size), int(refresh), float(softmax_scale))
    dev = q.device
    D = phi_dim(dqk)
    nblk = -(-T // refresh)
    o = torch.empty((B, Hh, T, dv), dtype=_torch_dtype(ocode), device=dev)
    HT = torch.empty((B, Hh, D, dv), dtype=torch.float32, device=dev) if return_state else None
    sT = torch.empty((B, Hh, D), dtype=torch.float32, device=dev) if return_state else None
    cT = torch.empty((B, Hh, cache_size), dtype=torch.int32, device=dev) if return_cache else None
    tr = torch.empty((B, Hh, nblk, cache_size), dtype=torch.int32, device=dev) if return_trace else None
    nbytes = ctypes.c_size_t(0)
    check(lib.kla_hybrid_workspace_size(ctypes.byref(shp), ctypes.byref(cfg), ctypes.byref(nbytes)))
    ws = _workspace(nbytes.value, dev)
    aux = None if aux_stream is None else ctypes.c_void_p(aux_stream.cuda_stream)
    check(lib.kla_hybrid_prefill_streams(ctypes.byref(shp), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(o), _ptr(HT), _ptr(sT), _ptr(cT), _ptr(tr), _ptr(ws),
                                         nbytes.value, _stream(dev), aux))
    if not (return_state or return_cache or return_trace):
        return o
    return o, dict(H=HT, s=sT, cache=cT, trace=tr)


def hybrid_decode_state(N: int, d_qk: int, d_v: int, window: int, cache_size: int, device, dtype=None):
    """Zeroed token-by-token hybrid state for N head-states: a dict of device
    tensors H [N, D, d_v], s [N, D], win_k [N, window+1, d_qk],
    win_v [N, window+1, d_v], cache_k [N, cache_size, d_qk],
    cache_v [N, cache_size, d_v], pend_k [N, P, d_qk], pend_v [N, P, d_v]
    (P = hybrid_decode_pending_slots()),
    cache_sums [N, cache_size, d_v + 4] (float32; numerators, denominator,
    padding) and cache_ids [N, cache_size] int32. The window and cache rows
    are in ``dtype`` (float32 or bfloat16, default float32), which must be
    the dtype of the tokens the steps take; everything else is float32."""
    torch = _torch()
    D = phi_dim(d_qk)
    P = hybrid_decode_pending_slots()
    f32 = dict(dtype=torch.float32, device=device)
    rdt = torch.float32 if dtype is None else dtype
    _dtype_code(torch.empty(0, dtype=rdt))  # float32 or bfloat16
    rows = dict(dtype=rdt, device=device)
    return dict(
        H=torch.zeros((N, D, d_v), **f32), s=torch.zeros((N, D), **f32),
        win_k=torch.zeros((N, window + 1, d_qk), **rows), win_v=torch.zeros((N, window + 1, d_v), **rows),
        cache_k=torch.zeros((N, cache_size, d_qk), **rows), cache_v=torch.zeros((N, cache_size, d_v), **rows),
        cache_ids=torch.full((N, cache_size), -1, dtype=torch.int32, device=device),
        pend_k=torch.zeros((N, P, d_qk), **f32), pend_v=torch.zeros((N, P, d_v), **f32),
        cache_sums=torch.zeros((N, cache_size, d_v + 4), **f32))


_STATE_FIELDS = ("H", "s", "win_k", "win_v", "cache_k", "cache_v", "cache_ids", "pend_k", "pend_v", "cache_sums")


def _hybrid_state_struct(state):
    for name in _STATE_FIELDS:
        t_ = state[name]
        if not t_.is_cuda or not t_.is_contiguous():
            raise TypeError(f"state['{name}'] must be a contiguous device tensor (updated in place)")
    return HybridState(*(state[n].data_ptr() for n in _STATE_FIELDS), _dtype_code(state["win_k"]))


def hybrid_decode_step(state, t: int, q, k, v, window: int, cache_size: int, softmax_scale=None,
                       eps: float = 0.0, out_dtype=None, rejected: bool = False, out=None, ws=None):
    """One token of the window + linear state + sparse cache decode for every
    head-state. ``state`` is the dict of hybrid_decode_state (updated in
    place); ``t`` is the number of tokens already seen; q, k [N, d_qk],
    v [N, d_v]. Returns o [N, d_v], or (o, rejected [N] int32) with
    ``rejected``. ``out`` / ``ws`` may pass a preallocated output and
    workspace (uint8 tensor)."""
    torch = _torch()
    lib = load_library()
    _need_device(q, k, v)
    st = _hybrid_state_struct(state)
    q, k, v = _dense(q), _dense(k), _dense(v)
    N, dqk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    cfg = HybridCfg(int(window), int(cache_size), 1, float(softmax_scale))
    dev = q.device
    o = out if out is not None else torch.empty((N, dv), dtype=_torch_dtype(ocode), device=dev)
    rej = torch.empty((N,), dtype=torch.int32, device=dev) if rejected else None
    nbytes = ctypes.c_size_t(0)
    check(lib.kla_hybrid_decode_workspace_size(N, dqk, dv, ctypes.byref(cfg), ctypes.byref(nbytes)))
    if ws is None or ws.numel() < nbytes.value:
        ws = _workspace(nbytes.value, dev)
    check(lib.kla_hybrid_decode_step(N, dqk, dv, float(eps), ctypes.byref(cfg), int(t), ctypes.byref(st),
                                     _ptr(q), _ptr(k), _ptr(v), code, _ptr(o), ocode, _ptr(rej), _ptr(ws),
                                     nbytes.value, _stream(dev)))
    return (o, rej) if rejected else o


def hybrid_decode_pending_slots() -> int:
    """Pending slots of a hybrid decode state: rejected pairs wait there and
    are folded into (H, s) together every that many tokens."""
    return int(load_library().kla_hybrid_decode_pending_slots())


def hybrid_decode_static_limit() -> int:
    """Bytes of the library's static scratch for hybrid_decode_step_static."""
    return int(load_library().kla_hybrid_decode_static_limit())


def hybrid_decode_step_static(state, t: int, q, k, v, window: int, cache_size: int, softmax_scale=None,
                              eps: float = 0.0, out_dtype=None, rejected: bool = False, out=None,
                              rejected_out=None):
    """hybrid_decode_step through the entry point that allocates nothing: its
    scratch is the library's static per-device array, so no workspace is
    passed. ``out`` / ``rejected_out`` may pass preallocated outputs; with
    both given (and contiguous, aligned inputs) this wrapper allocates
    nothing either. Calls that overlap on one device race."""
    torch = _torch()
    lib = load_library()
    _need_device(q, k, v)
    st = _hybrid_state_struct(state)
    q, k, v = _dense(q), _dense(k), _dense(v)
    N, dqk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    ocode = code if out_dtype is None else _dtype_code(torch.empty(0, dtype=out_dtype))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    cfg = HybridCfg(int(window), int(cache_size), 1, float(softmax_scale))
    dev = q.device
    o = out if out is not None else torch.empty((N, dv), dtype=_torch_dtype(ocode), device=dev)
    rej = None
    if rejected:
        rej = rejected_out if rejected_out is not None else torch.empty((N,), dtype=torch.int32, device=dev)
    check(lib.kla_hybrid_decode_step_static(N, dqk, dv, float(eps), ctypes.byref(cfg), int(t), ctypes.byref(st),
                                            _ptr(q), _ptr(k), _ptr(v), code, _ptr(o), ocode, _ptr(rej),
                                            _stream(dev)))
    return (o, rej) if rejected else o


def hybrid_decode_flush(state):
    """Fold the state's pending slots into (H, s) and zero them, so that H and
    s alone hold the linear memory."""
    lib = load_library()
    st = _hybrid_state_struct(state)
    N, _, dqk = state["pend_k"].shape
    dv = state["pend_v"].shape[-1]
    check(lib.kla_hybrid_decode_flush(N, dqk, dv, ctypes.byref(st), _stream(state["H"].device)))


def hybrid_decode_prime(state, t: int, window: int, cache_size: int):
    """Compute state['cache_sums'] from H, s, the pending slots and the cached
    keys, for a state filled from elsewhere (a prefill) that takes token t
    next."""
    lib = load_library()
    st = _hybrid_state_struct(state)
    N, _, dqk = state["pend_k"].shape
    dv = state["pend_v"].shape[-1]
    cfg = HybridCfg(int(window), int(cache_size), 1, 1.0)
    check(lib.kla_hybrid_decode_prime(N, dqk, dv, ctypes.byref(cfg), int(t), ctypes.byref(st),
                                      _stream(state["H"].device)))


def profile_enable(on: bool = True):
    """Record HIP events around each call's dominant kernel on this thread."""
    check(load_library().kla_profile_enable(int(bool(on))))


def profile_read():
    """(summed kernel milliseconds, kernels recorded, dropped) since the last read."""
    ms = ctypes.c_double(0)
    n = ctypes.c_int(0)
    dr = ctypes.c_int(0)
    check(load_library().kla_profile_read(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(dr)))
    return ms.value, n.value, dr.value
