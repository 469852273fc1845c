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
from tests.gpu_util import (DEV, FWD_TOL_BF16, GRAD_TOL_BF16, TOL_FP32, assert_close, dev, host,
                            rel_err, tols, torch_dtype)

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
    "fp16_small": (gi.Workload("hs", 0, 2, 6, 128, "fp16", seq="varlen", init_state=True,
                               final_state=True, seed=86), [300, 65, 7], None, L.GDN_ACT_SILU),
    "fp16_d32_mild": (gi.Workload("hm", 0, 2, 4, 32, "fp16", seq="varlen", init_state=True,
                                  final_state=True, seed=87), [129, 0, 64], (0.02, 0.3),
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
    tdt = torch_dtype(w.dtype)
    rf = gi.round_to(w.dtype)
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
    ft, gt = tols(w.dtype)
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


SPLIT_CASES = {
    # name: workload, lengths, cut per sequence (tokens in the first call), A range
    "bf16": (gi.Workload("sc", 0, 2, 4, 128, "bf16", seq="varlen", init_state=True,
                         final_state=True, seed=83), [300, 130, 5], [170, 2, 5], (0.02, 0.3)),
    "fp32": (gi.Workload("scf", 0, 1, 2, 32, "fp32", seq="varlen", init_state=True,
                         final_state=True, seed=84), [90, 40], [1, 37], (0.02, 0.3)),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_layer_split_and_continue(name):
    """A pack fed in two calls, each carrying the recurrent state and the
    conv state into the next (and, backward, their gradients back), against
    the oracle's single call over the whole pack: outputs and input
    gradients concatenate, parameter gradients add up, and the gradients of
    the initial states come out of the first call.  Cuts fall inside chunks
    and inside the conv window (a piece of 1 or 2 tokens)."""
    w, lens, cuts, A_range = SPLIT_CASES[name]
    inp = gi.make_inputs(w, seqlens=lens, A_range=A_range)
    bf = w.dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32
    rf = gi.round_bf16 if bf else None
    rng = np.random.default_rng(85)
    C = w.channels
    cs0 = rng.standard_normal((len(lens), 3, C)).astype(np.float32)
    dcs = rng.standard_normal((len(lens), 3, C)).astype(np.float32)
    if bf:
        cs0, dcs = gi.round_bf16(cs0), gi.round_bf16(dcs)
    cu = inp["cu_seqlens"]
    parts = []
    for first in (True, False):
        idx = np.concatenate([np.arange(cu[n], cu[n] + cuts[n]) if first else
                              np.arange(cu[n] + cuts[n], cu[n + 1]) for n in range(len(lens))])
        plens = [cuts[n] if first else lens[n] - cuts[n] for n in range(len(lens))]
        parts.append((idx, gi.cu_from_lengths(plens)))
    core = GDNCore(CoreConfig(hk=w.hk, hv=w.hv, d=w.d, dtype=tdt), device=DEV)

    def targs(idx, pcu):
        return (dev(inp["x"][idx], tdt), dev(inp["w_conv"]), dev(inp["a"][idx], tdt),
                dev(inp["b"][idx], tdt), dev(inp["A_log"]), dev(inp["dt_bias"]),
                dev(inp["z"][idx], tdt), dev(inp["w_norm"]), torch.from_numpy(pcu).to(DEV))

    a_args, b_args = targs(*parts[0]), targs(*parts[1])
    fa = core.forward(*a_args, S0=dev(inp["S0"]), want_final=True, conv_state=dev(cs0, tdt),
                      want_conv_state=True)
    fb = core.forward(*b_args, S0=fa["S_final"], want_final=True, conv_state=fa["conv_state_out"],
                      want_conv_state=True)
    ia, ib = parts[0][0], parts[1][0]
    gb = core.backward(fb, *b_args, dev(inp["dy"][ib], tdt), S0=fa["S_final"],
                       dS_final=dev(inp["dS_T"]), conv_state=fa["conv_state_out"],
                       d_conv_state=dev(dcs, tdt))
    ga = core.backward(fa, *a_args, dev(inp["dy"][ia], tdt), S0=dev(inp["S0"]), dS_final=gb["dS0"],
                       conv_state=dev(cs0, tdt), d_conv_state=gb["d_conv_state"])
    torch.cuda.synchronize()

    whole = dict(inp, conv_state=cs0, d_conv_state=dcs)
    sc = w.d ** -0.5
    rfw = oracle.layer_fwd(whole, w.hk, w.hv, w.d, sc, round_fn=rf)
    rbw = oracle.layer_bwd(whole, rfw, w.hk, w.hv, w.d, sc, round_fn=rf)
    order = np.argsort(np.concatenate([ia, ib]))

    def cat(k, a, b):
        return np.concatenate([host(a[k]).reshape(len(ia), -1), host(b[k]).reshape(len(ib), -1)])[order]

    ft = FWD_TOL_BF16 if bf else TOL_FP32
    gt = GRAD_TOL_BF16 if bf else TOL_FP32
    checks = [("out", cat("out", fa, fb), rfw["out"].reshape(len(order), -1), ft),
              ("S_final", host(fb["S_final"]), rfw["S_final"], ft),
              ("conv_state_out", host(fb["conv_state_out"]), rfw["conv_state_out"], ft),
              ("dx", cat("dx", ga, gb), rbw["dx"], gt),
              ("dz", cat("dz", ga, gb), rbw["dz"].reshape(len(order), -1), gt),
              ("da", cat("da", ga, gb), rbw["da"], gt), ("db", cat("db", ga, gb), rbw["db"], gt),
              ("dS0", host(ga["dS0"]), rbw["dS0"], gt),
              ("d_conv_state", host(ga["d_conv_state"]), rbw["d_conv_state"], gt)]
    for k in ("dw_conv", "dw_norm", "dA_log", "ddt_bias"):
        checks.append((k, host(ga[k]) + host(gb[k]), rbw[k], gt))
    errs = {k: rel_err(g_, r) for k, g_, r, _ in checks}
    print(name, " ".join(f"{k}={e:.2e}" for k, e in errs.items()), flush=True)
    for k, g_, r, tol in checks:
        assert_close(k, g_, r, tol)
