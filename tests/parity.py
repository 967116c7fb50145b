"""Comparison of the HIP path's output with the CPU oracle (test helper).

Acceptance, per head h over every compared (row, d):
  * max |O_gpu - O_oracle| <= 2e-2 over all compared elements,
  * cosine(O_gpu[:, h, :], O_oracle[:, h, :]) >= 0.9999 for every head,
  * |LSE_gpu - LSE_oracle| <= 1e-3 where the oracle's LSE is finite, and
    LSE_gpu == -inf exactly where the oracle's is (segments without keys),
  * no NaN or Inf in O.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 2e-2
MIN_COS = 0.9999
LSE_ABS = 1e-3


def compare(o_gpu, lse_gpu, o_ref, lse_ref, label=""):
    """o_*: [R, H, D]; lse_*: [R, H] (numpy, any float dtype). Returns stats; raises on failure."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    diff = np.abs(o_gpu - o_ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    rel = max_abs / max(float(np.abs(o_ref).max()) if o_ref.size else 0.0, 1e-30)
    R, H, D = o_ref.shape
    cos = []
    for h in range(H):
        a = o_gpu[:, h, :].ravel()
        b = o_ref[:, h, :].ravel()
        na, nb = np.linalg.norm(a), np.linalg.norm(b)
        if na == 0 and nb == 0:
            cos.append(1.0)
        elif na == 0 or nb == 0:
            cos.append(0.0)
        else:
            cos.append(float(np.dot(a, b) / (na * nb)))
    min_cos = min(cos) if cos else 1.0
    stats = {"max_abs": max_abs, "rel_max": rel, "min_cos": min_cos, "rows": R}
    assert max_abs <= MAX_ABS, f"{label}: max |dO| {max_abs:.3e} > {MAX_ABS}"
    assert min_cos >= MIN_COS, f"{label}: min per-head cosine {min_cos:.6f} < {MIN_COS}"
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        lr = np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lr)
        assert np.array_equal(np.isfinite(lg), fin), f"{label}: LSE finiteness differs"
        assert np.all(lg[~fin] == -np.inf), f"{label}: LSE of empty key segments must be -inf"
        dl = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
        stats["max_lse"] = dl
        assert dl <= LSE_ABS, f"{label}: max |dLSE| {dl:.3e} > {LSE_ABS}"
    return stats


# Gradients (dq, dk, dv) of the backward. The _bwd_preprocess page's repro
# script (its REL_TOL) accepts a gradient whose largest error is under 1e-2 of
# the reference's largest magnitude, which it treats as bf16 rounding; the
# per-head cosine bound is ours.
GRAD_REL = 1e-2
GRAD_COS = 0.9999


def compare_grad(g_gpu, g_ref, label=""):
    """g_*: [R, H, D] numpy. Relative max error against the reference's max
    magnitude, per-head cosine, finiteness. Returns stats; raises on failure."""
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    assert g_gpu.shape == g_ref.shape, (g_gpu.shape, g_ref.shape)
    assert np.all(np.isfinite(g_gpu)), f"{label}: non-finite gradient"
    scale = float(np.abs(g_ref).max()) if g_ref.size else 0.0
    err = float(np.abs(g_gpu - g_ref).max()) if g_ref.size else 0.0
    if scale == 0.0:
        assert err == 0.0, f"{label}: reference is zero but the gradient is not ({err:.3e})"
        return {"rel": 0.0, "min_cos": 1.0}
    rel = err / scale
    cos = []
    for h in range(g_ref.shape[1]):
        a, b = g_gpu[:, h].ravel(), g_ref[:, h].ravel()
        na, nb = np.linalg.norm(a), np.linalg.norm(b)
        cos.append(1.0 if na == 0 and nb == 0 else (0.0 if na == 0 or nb == 0 else float(a @ b / (na * nb))))
    stats = {"rel": rel, "min_cos": min(cos)}
    assert rel < GRAD_REL, f"{label}: max|dG|/max|G| {rel:.3e} >= {GRAD_REL}"
    assert min(cos) >= GRAD_COS, f"{label}: min per-head cosine {min(cos):.6f} < {GRAD_COS}"
    return stats
