"""Parity bars shared by the GPU tests.

Floating-point outputs: max |gpu - ref| <= 1e-2 * max |ref| and the mean
relative error sum|gpu - ref| / sum|ref| <= 2e-3; log-sum-exp values within
1e-3 absolute. Integer / byte work: bit-exact.
"""
import numpy as np

MAX_REL = 1e-2
L1_REL = 2e-3
LSE_ABS = 1e-3


def errors(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    err = np.abs(gpu - ref)
    return float(err.max() / max(np.abs(ref).max(), 1e-300)), float(err.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_bar(gpu, ref, what, max_rel=MAX_REL, l1_rel=L1_REL):
    mx, l1 = errors(gpu, ref)
    print(f"  {what}: max-rel {mx:.2e}  l1-rel {l1:.2e}", flush=True)
    assert mx <= max_rel, f"{what}: max error {mx:.3e} of max|ref| exceeds {max_rel}"
    assert l1 <= l1_rel, f"{what}: mean relative error {l1:.3e} exceeds {l1_rel}"
    return mx, l1


def assert_lse(gpu, ref, what, tol=LSE_ABS):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    same_inf = np.isneginf(gpu) == np.isneginf(ref)
    assert same_inf.all(), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    d = float(np.abs(gpu[fin] - ref[fin]).max()) if fin.any() else 0.0
    print(f"  {what}: max |dlse| {d:.2e}", flush=True)
    assert d <= tol, f"{what}: lse error {d:.3e} exceeds {tol}"
    return d
