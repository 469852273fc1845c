"""Helpers for GPU parity tests: host<->device copies and the error metric.

The error metric is the norm-wise max relative error of a tensor,
max|got - ref| / max|ref|, used for every floating-point comparison."""
import numpy as np
import torch

DEV = "cuda:0"
FWD_TOL_BF16 = 5e-3
GRAD_TOL_BF16 = 1e-2
TOL_FP32 = 1e-5
# 16-bit storage (bf16 or fp16) is held to the bf16 bars


def torch_dtype(dtype):
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]


def gdn_dtype(dtype):
    from gated_deltanet_layer_causal_amd import capi as L
    return {"bf16": L.GDN_BF16, "fp16": L.GDN_FP16, "fp32": L.GDN_FP32}[dtype]


def tols(dtype):
    """(forward, gradient) tolerance for a storage dtype"""
    return (TOL_FP32, TOL_FP32) if dtype == "fp32" else (FWD_TOL_BF16, GRAD_TOL_BF16)


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


FLOWS = ("composite", "saved")


def run_chunk(flow, sh, q, k, v, g, beta, scale, S0, cu, dout, dS_final, ws):
    """The chunked rule forward and backward through the C ABI, in one of the
    two flows: "composite" (gdn_chunk_fwd, then gdn_chunk_bwd, which
    recomputes the states) or "saved" (the training flow: backward-mode
    preparation, the state pass that saves the chunk states with the
    chunk-parallel outputs, then the reverse pass and the chunk gradients on
    that workspace).  Returns the device tensors o, S_final, dq, dk, dv, dg,
    dbeta, dS0 (dq, dk, dv as views into one [T, C] gradient tensor)."""
    from gated_deltanet_layer_causal_amd import capi as L
    T, n = sh.total_tokens, sh.n_seq
    hk, hv, d = sh.hk, sh.hv, sh.dk
    tdt = q.dtype
    Sf = torch.empty((n, hv, d, d), dtype=torch.float32, device=q.device)
    o = torch.empty((T, hv, d), dtype=tdt, device=q.device)
    dy = torch.empty((T, 2 * hk * d + hv * d), dtype=tdt, device=q.device)
    dq, dk, dv = dy[:, : hk * d], dy[:, hk * d: 2 * hk * d], dy[:, 2 * hk * d:]
    dg, db = torch.empty_like(g), torch.empty_like(beta)
    dS0 = torch.empty_like(Sf)
    if flow == "composite":
        L.gdn_chunk_fwd(sh, q, k, v, g, beta, scale, S0, Sf, cu, o, ws)
        L.gdn_chunk_bwd(sh, q, k, v, g, beta, scale, S0, cu, dout, dS_final, dq, dk, dv, dg, db,
                        dS0, ws)
    elif flow == "saved":
        L.gdn_chunk_prepare_bwd(sh, q, k, g, beta, scale, cu, ws)
        L.gdn_chunk_fwd_states_save(sh, q, k, v, scale, S0, Sf, cu, o, ws)
        L.gdn_chunk_bwd_reverse(sh, q, k, scale, cu, dout, dS_final, dv, dS0, ws)
        L.gdn_chunk_bwd_grads(sh, q, k, beta, scale, cu, dout, dv, dq, dk, dg, db, ws)
    else:
        raise ValueError(flow)
    return {"o": o, "S_final": Sf, "dq": dq, "dk": dk, "dv": dv, "dg": dg, "dbeta": db,
            "dS0": dS0}
