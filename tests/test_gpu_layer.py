"""Whole layer core (conv -> gate -> chunked gated delta rule -> gated norm,
forward and backward) on the GPU against the oracle's composed layer.

The oracle composition rounds to the storage dtype exactly at the tensors the
layer hands between its C-ABI calls (conv output, delta-rule output and the
gradients passed back), the interface values of the layer."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_layer_causal_amd import capi as L
from gated_deltanet_layer_causal_amd import inputs as gi
from gated_deltanet_layer_causal_amd.layer import CoreConfig, GDNCore, GDNLayer
from tests.gpu_util import DEV, FWD_TOL_BF16, GRAD_TOL_BF16, TOL_FP32, assert_close, dev, host, rel_err

pytestmark = pytest.mark.gpu

CASES = {
    # name: workload, seqlens, A range, activation
    "tiny_fp32": (gi.WORKLOADS["tiny"], [64], None, L.GDN_ACT_SILU),
    "tiny_fp32_varlen_state": (gi.Workload("tv", 0, 1, 2, 32, "fp32", seq="varlen",
                                           init_state=True, final_state=True, seed=77),
                               [40, 1, 90], (0.02, 0.3), L.GDN_ACT_SIGMOID),
    "bf16_small": (gi.Workload("bs", 0, 2, 6, 128, "bf16", seq="varlen", init_state=True,
                               final_state=True, seed=78), [300, 65, 7], None, L.GDN_ACT_SILU),
    # empty sequences inside and at the end of the pack: their state passes
    # through unchanged and so does its gradient
    "bf16_empty_seqs": (gi.Workload("be", 0, 2, 4, 128, "bf16", seq="varlen", init_state=True,
                                    final_state=True, seed=79), [70, 0, 64, 0, 5], None,
                        L.GDN_ACT_SILU),
    "fp32_empty_first": (gi.Workload("fe", 0, 1, 2, 32, "fp32", seq="varlen", init_state=True,
                                     final_state=True, seed=80), [0, 40, 0, 3], (0.02, 0.3),
                         L.GDN_ACT_SIGMOID),
}


@pytest.mark.parametrize("seg", [0, 2], ids=["seq", "seg2"])
@pytest.mark.parametrize("save_states", [True, False], ids=["saved", "recompute"])
@pytest.mark.parametrize("name", list(CASES))
def test_layer_matches_oracle(name, save_states, seg):
    """Both backward flows: states saved by the forward, or recomputed; one
    sequential pass per sequence, or the segment-parallel scan with segments
    of two chunks."""
    w, lens, A_range, act = CASES[name]
    inp = gi.make_inputs(w, seqlens=lens, A_range=A_range)
    bf = w.dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32
    rf = gi.round_bf16 if bf else None
    core = GDNCore(CoreConfig(hk=w.hk, hv=w.hv, d=w.d, dtype=tdt, act=act, seg_chunks=seg),
                   device=DEV)
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    args = (dev(inp["x"], tdt), dev(inp["w_conv"]), dev(inp["a"], tdt), dev(inp["b"], tdt),
            dev(inp["A_log"]), dev(inp["dt_bias"]), dev(inp["z"], tdt), dev(inp["w_norm"]), cu)
    S0 = dev(inp["S0"]) if inp["S0"] is not None else None
    dST = dev(inp["dS_T"]) if inp["dS_T"] is not None else None
    f = core.forward(*args, S0=S0, want_final=True, save_states=save_states)
    gb = core.backward(f, *args, dev(inp["dy"], tdt), S0=S0, dS_final=dST)
    torch.cuda.synchronize()
    sc = w.d ** -0.5
    rf_ = f_ = oracle.layer_fwd(inp, w.hk, w.hv, w.d, sc, act=act, round_fn=rf)
    rb = oracle.layer_bwd(inp, rf_, w.hk, w.hv, w.d, sc, act=act, round_fn=rf)
    ft = TOL_FP32 if not bf else FWD_TOL_BF16
    gt = TOL_FP32 if not bf else GRAD_TOL_BF16
    checks = [(k, f[k], f_[k], ft) for k in ("y", "g", "beta", "o", "out", "S_final")]
    checks += [(k, gb[k], rb[k], gt) for k in ("do", "dg", "dbeta", "dy_conv", "dx", "dw_conv", "da",
                                               "db", "dA_log", "ddt_bias", "dz", "dw_norm", "dS0")]
    # every error is printed before the first assertion, so a failure shows
    # where along the layer the difference enters
    errs = {k: rel_err(host(t).reshape(np.shape(r)), r) for k, t, r, _ in checks}
    print(name, "saved" if save_states else "recompute", f"seg={seg}", " ".join(f"{k}={e:.2e}" for k, e in errs.items()), flush=True)
    for k, t, r, tol in checks:
        assert_close(k, host(t).reshape(np.shape(r)), r, tol)
    # a sequence without tokens hands its initial state and the final state's
    # gradient straight through (exactly: no arithmetic touches them)
    for n, ln in enumerate(lens):
        if ln == 0:
            np.testing.assert_array_equal(host(f["S_final"])[n], np.float32(inp["S0"][n]))
            np.testing.assert_array_equal(host(gb["dS0"])[n], np.float32(inp["dS_T"][n]))


def test_layer_with_projections_matches_oracle():
    """The layer with its in/out projections (library GEMMs around libgdn)
    against the oracle's composition (fp64 products around the core oracle,
    rounded to bf16 where the layer hands tensors between calls)."""
    hk, hv, d, H = 2, 4, 128, 256
    w = gi.Workload("pl", 0, hk, hv, d, "bf16", seq="varlen", init_state=True, final_state=True,
                    seed=81)
    lens = [150, 64, 1]
    inp = gi.make_inputs(w, seqlens=lens)
    T = sum(lens)
    rng = np.random.default_rng(82)
    rb = gi.round_bf16
    X = rb(rng.standard_normal((T, H)).astype(np.float32))
    shapes = {"x": (w.channels, H), "z": (hv * d, H), "a": (hv, H), "b": (hv, H), "out": (H, hv * d)}
    W = {k: rb((rng.standard_normal(s) / np.sqrt(s[1])).astype(np.float32)) for k, s in shapes.items()}
    dY = rb(rng.standard_normal((T, H)).astype(np.float32))
    params = {k: inp[k] for k in ("w_conv", "A_log", "dt_bias", "w_norm")}
    bf = torch.bfloat16
    layer = GDNLayer(CoreConfig(hk=hk, hv=hv, d=d, dtype=bf), H, {k: dev(v, bf) for k, v in W.items()},
                     device=DEV)
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    gargs = (dev(params["w_conv"]), dev(params["A_log"]), dev(params["dt_bias"]), dev(params["w_norm"]), cu)
    S0, dST = dev(inp["S0"]), dev(inp["dS_T"])
    f = layer.forward(dev(X, bf), *gargs, S0=S0, want_final=True)
    g = layer.backward(f, dev(X, bf), *gargs, dev(dY, bf), S0=S0, dS_final=dST)
    torch.cuda.synchronize()

    sc = d ** -0.5
    rf_ = oracle.proj_layer_fwd(X, W, params, inp["cu_seqlens"], hk, hv, d, sc, round_fn=rb,
                                S0=inp["S0"])
    rg = oracle.proj_layer_bwd(X, W, rf_, dY, hk, hv, d, sc, round_fn=rb, dS_T=inp["dS_T"])
    checks = [("Y", f["Y"], rf_["Y"], FWD_TOL_BF16), ("S_final", f["S_final"], rf_["S_final"], FWD_TOL_BF16),
              ("dX", g["dX"], rg["dX"], GRAD_TOL_BF16), ("dS0", g["dS0"], rg["dS0"], GRAD_TOL_BF16),
              ("dw_conv", g["dw_conv"], rg["dw_conv"], GRAD_TOL_BF16),
              ("dA_log", g["dA_log"], rg["dA_log"], GRAD_TOL_BF16),
              ("ddt_bias", g["ddt_bias"], rg["ddt_bias"], GRAD_TOL_BF16),
              ("dw_norm", g["dw_norm"], rg["dw_norm"], GRAD_TOL_BF16)]
    checks += [(f"dW_{k}", g["dW"][k], rg["dW"][k], GRAD_TOL_BF16) for k in W]
    errs = {k: rel_err(host(t).reshape(np.shape(r)), r) for k, t, r, _ in checks}
    print("projections", " ".join(f"{k}={e:.2e}" for k, e in errs.items()), flush=True)
    for k, t, r, tol in checks:
        assert_close(k, host(t).reshape(np.shape(r)), r, tol)
