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


def assert_update_parity(y, ref, x, dtype, what=""):
    """Parity of the block update x_out - x_in.

    A bf16 output carries its own rounding (up to half an ulp of x_out),
    which no implementation can avoid; when the update is small next to x
    that floor alone can exceed the bare criterion.  The bound is therefore
    the method's tolerance on top of the floor measured for the exactly
    rounded oracle output: max-abs <= 2e-2 + floor and
    1 - cos <= 1e-4 + 2 (1 - cos_floor).  For fp32 the floor is ~0 and the
    bare fp32 criterion applies."""
    x = np.asarray(x, np.float64)
    if dtype == "f32":
        return assert_parity(y - x, ref - x, "f32", what)
    ferr, fcos = metrics(bf16_nearest(ref) - x, ref - x)
    return assert_parity(y - x, ref - x, "bf16", f"{what} (floor {ferr:.2e}/{fcos:.6f})",
                         maxabs=BF16_MAXABS + ferr, cos_min=1 - (1 - BF16_COS) - 2 * (1 - fcos))
