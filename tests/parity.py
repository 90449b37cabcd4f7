"""Comparison helpers for the GPU parity tests (tolerances of the layer contract)."""
import numpy as np
import torch

REL_L2 = 2e-3          # relative L2 error bound for floating-point outputs
MAX_ABS_FRAC = 1e-2    # max-abs error bound, as a fraction of max |reference|


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.numpy()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def assert_close(got, ref, rel=REL_L2, max_abs_frac=MAX_ABS_FRAC, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    r = rel_l2(got, ref)
    m = float(np.abs(got - ref).max()) if got.size else 0.0
    lim = max_abs_frac * float(np.abs(ref).max()) if ref.size else 0.0
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel:.1e}"
    assert m <= lim, f"{what}: max-abs {m:.3e} > {lim:.3e}"
    return r, m
