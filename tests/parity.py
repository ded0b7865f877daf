"""Error measure shared by the GPU parity tests, and one input shaping helper.

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


def stepped_scores(q, k, n_rep, step=0.6, seed=5):
    """Queries and keys whose scores climb by about 10 (log2 units, at head_dim 128 and the
    default scale) from one 64-key tile to the next: every key of KV head g points along one
    direction u_g (the group's queries too), times 1 + step * (position // 64), plus 10% noise.
    Every later tile then lifts the running max by more than the kernel's 2^8 slack, so the
    reference max moves (scores shifted, O and l rescaled) tile after tile, while keys of one
    tile stay close, so the rows stay smooth averages of V.  Callers keep to about 7 tiles:
    the scores then stay below about 75, where the bf16-rounded scaled query (relative score
    error about 2^-9 / sqrt(head_dim)) moves the weights by well under the 2e-2 tolerance.
    NaN entries of q and k stay NaN."""
    import torch

    g = torch.Generator().manual_seed(seed)
    B, S, Hq, D = q.shape
    T, Hkv = k.shape[1], k.shape[2]
    u = torch.randn(B, 1, Hkv, D, generator=g)
    qu = u.repeat_interleave(n_rep, dim=2)  # the contiguous head grouping: head h uses u_(h // n_rep)
    qn = qu + 0.1 * torch.randn(B, S, Hq, D, generator=g)
    mag = 1.0 + step * (torch.arange(T) // 64).float()
    kn = mag[None, :, None, None] * (u + 0.1 * torch.randn(B, T, Hkv, D, generator=g))
    return (q.float() * 0 + qn).to(q.dtype), (k.float() * 0 + kn).to(k.dtype)
