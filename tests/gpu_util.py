"""Helpers for GPU parity tests: host<->device copies and the error metric.

The error metric is the norm-wise max relative error of a tensor,
max|got - ref| / max|ref|, used for every floating-point comparison."""
import numpy as np
import torch

DEV = "cuda:0"
FWD_TOL_BF16 = 5e-3
GRAD_TOL_BF16 = 1e-2
TOL_FP32 = 1e-5


def dev(a, dtype=torch.float32):
    """numpy -> device tensor; bf16-exact float32 input converts exactly."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: max rel err {e:.3e} > {tol:.1e}"
    return e
