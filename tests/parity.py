"""Error measure shared by the GPU parity tests.

Max relative error, normwise per output row: for each row (one (b, h) of a decode, one
(b, i, h) of a prefill) max_d |gpu - ref| / max_d |ref|; a case passes when its worst row is
within the tolerance.  Elementwise relative error is not used because outputs near zero make
it meaningless.  An all-zero reference row (an empty cache) must be matched exactly."""
import numpy as np

TOL_FP32 = 1e-5   # fp32 inputs
TOL_BF16 = 2e-2   # bf16 inputs, fp32 accumulation


def to_np(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_err(gpu, ref) -> float:
    g, r = to_np(gpu), to_np(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    D = g.shape[-1]
    g2, r2 = g.reshape(-1, D), r.reshape(-1, D)
    if not np.all(np.isfinite(g2)):
        return float("inf")
    num = np.max(np.abs(g2 - r2), axis=1)
    den = np.max(np.abs(r2), axis=1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float(np.max(num[~zero] / den[~zero]))


def assert_close_rows(gpu, ref, tol, what=""):
    err = row_rel_err(gpu, ref)
    print(f"[parity] {what}: worst-row relative error {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{what}: worst-row relative error {err:.3e} > {tol:.0e}"
    return err
