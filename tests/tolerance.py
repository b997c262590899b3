"""Comparison rules shared by the parity tests.

Floating point: elementwise |x - r| <= rtol * (|r| + rho), with rho the RMS of
the reference over the compared tensor. The floor rho is needed because an
attention output is a convex mix of signed values, so single entries can
cancel to about zero while their rounding error scales with the terms.
rtol is 1e-4 for fp32 paths and 2e-2 for bf16-input paths.

Top-k sets: exact when the oracle's boundary gap exceeds 1e-5 relative;
otherwise any set that keeps only near-boundary scores and every clearly
larger one is accepted (oracle.near_tie_ok).
"""
import numpy as np

RTOL_F32 = 1e-4
RTOL_BF16 = 2e-2
TIE_REL = 1e-5


def rel_report(x, r):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    rho = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(x - r)
    scaled = err / (np.abs(r) + rho + 1e-300)
    nrm = float(np.linalg.norm(x - r) / (np.linalg.norm(r) + 1e-300))
    return dict(max_scaled=float(scaled.max()) if r.size else 0.0, normwise=nrm, rho=rho,
                worst=int(np.argmax(scaled)) if r.size else -1)


def assert_close(x, r, rtol, what="tensor"):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, f"{what}: shape {x.shape} vs {r.shape}"
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    rep = rel_report(x, r)
    assert rep["max_scaled"] <= rtol, (
        f"{what}: max |x-r|/(|r|+rho) = {rep['max_scaled']:.3e} > {rtol:.1e} "
        f"(normwise {rep['normwise']:.3e}, rho {rep['rho']:.3e}, flat index {rep['worst']}, "
        f"x={x.reshape(-1)[rep['worst']]!r}, r={r.reshape(-1)[rep['worst']]!r})")
    return rep
