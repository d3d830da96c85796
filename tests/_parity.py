"""Parity criteria shared by the GPU tests.

bf16 path: max|y - ref| <= 2e-2 * max|ref| and cos(y, ref) >= 0.9999.
fp32 path: max|y - ref| <= 1e-4 * max|ref|.
Applied to block outputs and to the block update x_out - x_in.
"""
import numpy as np

BF16_MAXABS, BF16_COS, F32_REL = 2e-2, 0.9999, 1e-4


def metrics(y, ref):
    y = np.asarray(y, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(y - ref)) / scale if scale > 0 else np.max(np.abs(y - ref))
    den = np.linalg.norm(y) * np.linalg.norm(ref)
    cos = float(y @ ref / den) if den > 0 else (1.0 if np.all(y == ref) else 0.0)
    return float(err), cos


def assert_parity(y, ref, dtype, what="", maxabs=None, cos_min=None):
    err, cos = metrics(y, ref)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if dtype == "f32":
        tol = F32_REL if maxabs is None else maxabs
        assert err <= tol, f"{what}: max-abs/max|ref| = {err:.3e} > {tol:.1e}"
    else:
        tol = BF16_MAXABS if maxabs is None else maxabs
        cmin = BF16_COS if cos_min is None else cos_min
        assert err <= tol and cos >= cmin, f"{what}: max-abs/max|ref| = {err:.3e} (<= {tol:.1e}), cos = {cos:.7f} (>= {cmin})"
    return err, cos


def bf16_nearest(a):
    """float64 -> nearest bf16 value (via float32), as float64."""
    import datagen
    return datagen.bf16_round(np.asarray(a, np.float32)).astype(np.float64)


def half_ulp_bf16(a):
    """Half the bf16 spacing at |a| (the largest rounding error of a value of that size)."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def assert_update_parity(y, ref, x, dtype, what="", maxabs=None, cos_min=None):
    """Parity of the block update x_out - x_in.

    A bf16 output carries its own rounding (up to half a bf16 ulp of each
    x_out element), which no implementation avoids; when the update is
    small next to x that rounding alone can exceed the bare criterion.  So
    each element's error is first reduced by that half ulp, and the rest
    must be within the method's bound: max(|dy - dref| - ulp/2) <= 2e-2 *
    max|dref|; and 1 - cos <= 1e-4 + 2 (1 - cos_floor), cos_floor being the
    cosine reached by the exactly rounded oracle output.  maxabs and
    cos_min replace the 2e-2 and 0.9999 of that criterion (a path with a
    wider derived bound, such as the 8-bit one).  For fp32 the bare fp32
    criterion applies."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if dtype == "f32":
        return assert_parity(y - x, ref - x, "f32", what)
    dy, dr = y - x, ref - x
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    excess = np.max(np.maximum(np.abs(dy - dr) - np.maximum(half_ulp_bf16(ref), half_ulp_bf16(y)), 0.0))
    scale = np.max(np.abs(dr))
    err = excess / scale
    _, fcos = metrics(bf16_nearest(ref) - x, dr)
    _, cos = metrics(dy, dr)
    tol = BF16_MAXABS if maxabs is None else maxabs
    cmin = 1 - (1 - (BF16_COS if cos_min is None else cos_min)) - 2 * (1 - fcos)
    assert err <= tol and cos >= cmin, (
        f"{what}: max(|d-dref| - ulp/2)/max|dref| = {err:.3e} (<= {tol:.0e}), "
        f"cos = {cos:.7f} (>= {cmin:.7f}, floor {fcos:.7f})")
    return err, cos
