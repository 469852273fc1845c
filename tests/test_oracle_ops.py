"""Pins for the oracle's conv, gate and gated norm, and the composed layer
(CPU only): hand-worked values, textbook/library routines, invariants and
finite differences."""
import os

import numpy as np
import pytest
import scipy.special as sp
import torch
import torch.nn.functional as F

import oracle
from gated_deltanet_layer_causal_amd import inputs as gi

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ conv
def test_conv_hand_worked():
    rows = {}
    for line in open(os.path.join(GOLD, "conv_hand_5tok.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            parts = line.split()
            rows[parts[0]] = np.array([float(x) for x in parts[1:]])
    x = np.arange(1.0, 6.0).reshape(5, 1)
    w = np.array([[0.5, 0.0, -1.0, 2.0]])
    for case, cu in (("single", [0, 5]), ("split", [0, 2, 5])):
        y = oracle.conv_fwd(x, w, cu, 0, 1)
        u = rows[case]
        np.testing.assert_allclose(y[:, 0], u * sp.expit(u), rtol=1e-15)


def test_conv_matches_numpy_convolve_and_l2():
    """I8: per channel, the pre-activation equals numpy.convolve(x_c, w_c[::-1])[:L]
    restarted at every sequence; q/k heads are then unit-normalised."""
    rng = np.random.default_rng(0)
    hk, hv, d = 2, 3, 4
    C = 2 * hk * d + hv * d
    lens = [9, 2, 14]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = cu[-1]
    x = rng.standard_normal((T, C))
    w = 0.25 * rng.standard_normal((C, 4))
    y = oracle.conv_fwd(x, w, cu, 2 * hk * d, d, eps=1e-6)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        u = np.stack([np.convolve(x[a:b, c], w[c, ::-1])[: b - a] for c in range(C)], axis=1)
        act = u * sp.expit(u)
        qk = act[:, : 2 * hk * d].reshape(b - a, 2 * hk, d)
        nrm = np.sqrt((np.linalg.norm(qk, axis=-1, keepdims=True)) ** 2 + 1e-6)
        ref = np.concatenate([(qk / nrm).reshape(b - a, -1), act[:, 2 * hk * d:]], axis=1)
        np.testing.assert_allclose(y[a:b], ref, rtol=1e-12, atol=1e-14)
    # q/k heads have unit norm up to eps
    nr = np.linalg.norm(y[:, : 2 * hk * d].reshape(T, 2 * hk, d), axis=-1)
    assert np.all(nr <= 1.0) and np.all(nr > 0.9)


def test_conv_permutation_equivariant_over_heads():
    """Permuting whole heads of the input permutes the output the same way
    (the channel layout is a permutation only)."""
    rng = np.random.default_rng(1)
    hk, d = 3, 4
    C = 2 * hk * d
    x = rng.standard_normal((11, C))
    w = rng.standard_normal((C, 4))
    perm_heads = np.array([2, 0, 1, 4, 5, 3])
    perm = (perm_heads[:, None] * d + np.arange(d)).reshape(-1)
    y = oracle.conv_fwd(x, w, [0, 11], C, d)
    yp = oracle.conv_fwd(x[:, perm], w[perm], [0, 11], C, d)
    np.testing.assert_array_equal(yp, y[:, perm])


# ------------------------------------------------------------------ gate
def test_gate_closed_form():
    """g = -exp(A_log) softplus(a + dt_bias) with A_log = log A (Megatron page,
    review: A_log stores log(A)); beta = sigmoid(b)."""
    rng = np.random.default_rng(2)
    T, H = 50, 5
    a = 4 * rng.standard_normal((T, H))
    a[0, 0], a[1, 0] = 60.0, -60.0
    b = 3 * rng.standard_normal((T, H))
    A = rng.uniform(1, 16, H)
    dt = rng.standard_normal(H)
    g, beta = oracle.gate_fwd(a, b, np.log(A), dt)
    np.testing.assert_allclose(g, -A * np.logaddexp(0.0, a + dt), rtol=1e-14)
    np.testing.assert_allclose(beta, sp.expit(b), rtol=1e-15)
    assert np.all(g < 0)


def test_gate_backward_finite_differences():
    rng = np.random.default_rng(3)
    T, H = 7, 3
    a, b = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    Al, dt = np.log(rng.uniform(1, 16, H)), rng.standard_normal(H)
    dg, dbeta = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    da, db, dAl, ddt = oracle.gate_bwd(a, b, Al, dt, dg, dbeta)

    def L(a_, b_, Al_, dt_):
        g, be = oracle.gate_fwd(a_, b_, Al_, dt_)
        return float((g * dg).sum() + (be * dbeta).sum())

    h = 1e-6
    for name, grad, idx in (("a", da, 0), ("b", db, 1), ("A_log", dAl, 2), ("dt", ddt, 3)):
        base = [a, b, Al, dt]
        num = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            p, m = [x.copy() for x in base], [x.copy() for x in base]
            p[idx][i] += h
            m[idx][i] -= h
            num[i] = (L(*p) - L(*m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-8, err_msg=name)


# ------------------------------------------------------------------ gated norm
@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_SIGMOID])
def test_norm_matches_torch_rms_norm(act):
    """Zero-centred RMSNorm (Megatron page: --apply-layernorm-1p; prime-rl page:
    ZeroCenteredRMSNorm) scales by (1 + w); the gate's activation is a kwarg
    (prime-rl page: "silu"/"sigmoid")."""
    rng = np.random.default_rng(4)
    o = rng.standard_normal((13, 3, 16))
    z = rng.standard_normal((13, 3, 16))
    w = 0.1 * rng.standard_normal(16)
    y = oracle.norm_fwd(o, z, w, act)
    ot = torch.from_numpy(o)
    ref = F.rms_norm(ot, (16,), weight=torch.from_numpy(1.0 + w), eps=1e-6)
    zt = torch.from_numpy(z)
    ref = ref * (F.silu(zt) if act == oracle.ACT_SILU else torch.sigmoid(zt))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_norm_plain_rmsnorm_and_scale_invariance():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((20, 32))
    z = np.full_like(o, 800.0)           # sigmoid(z) == 1 in double
    y = oracle.norm_fwd(o, z, np.zeros(32), oracle.ACT_SIGMOID, eps=0.0)
    rms = np.sqrt((o ** 2).mean(axis=1, keepdims=True))
    np.testing.assert_allclose(y, o / rms, rtol=1e-14)
    y2 = oracle.norm_fwd(7.5 * o, z, np.zeros(32), oracle.ACT_SIGMOID, eps=0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-14)


@pytest.mark.parametrize("act", [oracle.ACT_SILU, oracle.ACT_SIGMOID])
def test_norm_backward_finite_differences(act):
    rng = np.random.default_rng(6)
    o, z = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    w, dy = 0.1 * rng.standard_normal(6), rng.standard_normal((4, 6))
    do, dz, dw = oracle.norm_bwd(o, z, w, dy, act)

    def L(o_, z_, w_):
        return float((oracle.norm_fwd(o_, z_, w_, act) * dy).sum())

    h = 1e-6
    for name, grad, idx in (("o", do, 0), ("z", dz, 1), ("w", dw, 2)):
        base = [o, z, w]
        num = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            p, m = [x.copy() for x in base], [x.copy() for x in base]
            p[idx][i] += h
            m[idx][i] -= h
            num[i] = (L(*p) - L(*m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-8, err_msg=name)


# ------------------------------------------------------------------ conv backward
def test_conv_backward_finite_differences():
    rng = np.random.default_rng(7)
    hk, hv, d = 1, 1, 3
    C = 2 * hk * d + hv * d
    lens = [5, 3]
    cu = np.array([0, 5, 8], dtype=np.int32)
    x = rng.standard_normal((8, C))
    w = 0.5 * rng.standard_normal((C, 4))
    dy = rng.standard_normal((8, C))
    dx, dw = oracle.conv_bwd(x, w, cu, 2 * hk * d, d, dy)

    def L(x_, w_):
        return float((oracle.conv_fwd(x_, w_, cu, 2 * hk * d, d) * dy).sum())

    h = 1e-6
    for name, grad, idx in (("x", dx, 0), ("w", dw, 1)):
        base = [x, w]
        num = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            p, m = [a.copy() for a in base], [a.copy() for a in base]
            p[idx][i] += h
            m[idx][i] -= h
            num[i] = (L(*p) - L(*m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-8, err_msg=name)


# ------------------------------------------------------------------ conv with a carried state
def _state_case(seed, lens, hk=2, hv=3, d=4):
    rng = np.random.default_rng(seed)
    C = 2 * hk * d + hv * d
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    x = rng.standard_normal((T, C))
    w = 0.3 * rng.standard_normal((C, 4))
    cs = rng.standard_normal((len(lens), 3, C))
    return x, w, cu, cs, 2 * hk * d, d


def test_conv_state_zero_equals_stateless():
    """No state (or a zero state) is the stateless convolution, exactly."""
    x, w, cu, cs, n_l2, d = _state_case(30, [9, 1, 0, 14])
    y0 = oracle.conv_fwd(x, w, cu, n_l2, d)
    for cs_in in (None, np.zeros_like(cs)):
        y, _ = oracle.conv_state_fwd(x, w, cu, n_l2, d, cs_in)
        np.testing.assert_array_equal(y, y0)
    dy = np.random.default_rng(31).standard_normal(x.shape)
    dx0, dw0 = oracle.conv_bwd(x, w, cu, n_l2, d, dy)
    dx, dw, _ = oracle.conv_state_bwd(x, w, cu, n_l2, d, dy)
    np.testing.assert_allclose(dx, dx0, rtol=1e-15, atol=0)
    np.testing.assert_allclose(dw, dw0, rtol=1e-14, atol=1e-15)


def test_conv_state_matches_numpy_convolve_with_state_prepended():
    """Per channel the pre-activation is numpy.convolve over the state rows
    followed by the sequence (the state stands for the three inputs before
    it), and the final state is the last three inputs of that extended
    sequence (reaching into the initial state for sequences shorter than
    three)."""
    x, w, cu, cs, n_l2, d = _state_case(32, [9, 2, 0, 1, 14])
    y, cs_out = oracle.conv_state_fwd(x, w, cu, n_l2, d, cs)
    C = x.shape[1]
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        ext = np.concatenate([cs[n], x[a:b]], axis=0)            # [3 + L, C]
        u = np.stack([np.convolve(ext[:, c], w[c, ::-1])[3: 3 + b - a] for c in range(C)], axis=1)
        act = u * sp.expit(u)
        qk = act[:, :n_l2].reshape(b - a, n_l2 // d, d)
        nrm = np.sqrt((np.linalg.norm(qk, axis=-1, keepdims=True)) ** 2 + 1e-6)
        ref = np.concatenate([(qk / nrm).reshape(b - a, n_l2), act[:, n_l2:]], axis=1)
        np.testing.assert_allclose(y[a:b], ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(cs_out[n], ext[-3:])


@pytest.mark.parametrize("cut", [1, 2, 3, 7])
def test_conv_state_continuation(cut):
    """Splitting every sequence after `cut` tokens and feeding the first
    call's final state to the second call reproduces the whole call: outputs
    and final state exactly, and backward (the second call's state gradient
    fed back as the first call's final-state gradient) the input and state
    gradients, with dw the sum of the two calls'."""
    lens = [12, 9, 15]
    x, w, cu, cs, n_l2, d = _state_case(33 + cut, lens)
    rng = np.random.default_rng(40 + cut)
    dy = rng.standard_normal(x.shape)
    dcs = rng.standard_normal(cs.shape)
    y, cs_out = oracle.conv_state_fwd(x, w, cu, n_l2, d, cs)
    dx, dw, dcs_in = oracle.conv_state_bwd(x, w, cu, n_l2, d, dy, cs, dcs)
    ia = np.concatenate([np.arange(cu[n], cu[n] + cut) for n in range(len(lens))])
    ib = np.concatenate([np.arange(cu[n] + cut, cu[n + 1]) for n in range(len(lens))])
    cua = np.arange(len(lens) + 1, dtype=np.int32) * cut
    cub = np.concatenate([[0], np.cumsum([ln - cut for ln in lens])]).astype(np.int32)
    ya, csa = oracle.conv_state_fwd(x[ia], w, cua, n_l2, d, cs)
    yb, csb = oracle.conv_state_fwd(x[ib], w, cub, n_l2, d, csa)
    np.testing.assert_array_equal(np.concatenate([ya, yb])[np.argsort(np.concatenate([ia, ib]))], y)
    np.testing.assert_array_equal(csb, cs_out)
    dxb, dwb, dcsb = oracle.conv_state_bwd(x[ib], w, cub, n_l2, d, dy[ib], csa, dcs)
    dxa, dwa, dcsa = oracle.conv_state_bwd(x[ia], w, cua, n_l2, d, dy[ia], cs, dcsb)
    np.testing.assert_allclose(np.concatenate([dxa, dxb])[np.argsort(np.concatenate([ia, ib]))], dx,
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dcsa, dcs_in, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dwa + dwb, dw, rtol=1e-12, atol=1e-12)


def test_conv_state_backward_finite_differences():
    x, w, cu, cs, n_l2, d = _state_case(34, [5, 1, 0, 3], hk=1, hv=1, d=3)
    rng = np.random.default_rng(35)
    dy = rng.standard_normal(x.shape)
    dcs = rng.standard_normal(cs.shape)
    dx, dw, dcs_in = oracle.conv_state_bwd(x, w, cu, n_l2, d, dy, cs, dcs)

    def L(x_, w_, cs_):
        y, co = oracle.conv_state_fwd(x_, w_, cu, n_l2, d, cs_)
        return float((y * dy).sum() + (co * dcs).sum())

    h = 1e-6
    for name, grad, idx in (("x", dx, 0), ("w", dw, 1), ("cs_in", dcs_in, 2)):
        base = [x, w, cs]
        num = np.zeros_like(grad)
        for i in np.ndindex(grad.shape):
            p, m = [a.copy() for a in base], [a.copy() for a in base]
            p[idx][i] += h
            m[idx][i] -= h
            num[i] = (L(*p) - L(*m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-7, atol=1e-8, err_msg=name)


# ------------------------------------------------------------------ whole layer
def test_layer_backward_finite_differences():
    """Directional central differences through conv -> gate -> delta -> norm
    for every layer input (x, w_conv, a, b, A_log, dt_bias, z, w_norm, S0)."""
    w = gi.Workload("fd", 10, 1, 2, 4, "fp32", seq="varlen", init_state=True, final_state=True,
                    seed=5)
    inp = gi.make_inputs(w, seqlens=[6, 4], A_range=(0.05, 0.5))
    inp = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) and v.dtype == np.float32 else v)
           for k, v in inp.items()}
    hk, hv, d, sc = 1, 2, 4, 0.5
    fwd = oracle.layer_fwd(inp, hk, hv, d, sc)
    bwd = oracle.layer_bwd(inp, fwd, hk, hv, d, sc)

    def L(key, val):
        x = dict(inp)
        x[key] = val
        f = oracle.layer_fwd(x, hk, hv, d, sc)
        return float((f["out"] * inp["dy"]).sum() + (f["S_final"] * inp["dS_T"]).sum())

    rng = np.random.default_rng(8)
    pairs = (("x", "dx"), ("w_conv", "dw_conv"), ("a", "da"), ("b", "db"), ("A_log", "dA_log"),
             ("dt_bias", "ddt_bias"), ("z", "dz"), ("w_norm", "dw_norm"), ("S0", "dS0"))
    # z's gradient is dz from the norm; layer_bwd reports it under "dz"
    for key, gkey in pairs:
        x0 = inp[key]
        for _ in range(2):
            u = rng.standard_normal(x0.shape)
            h = 1e-6
            num = (L(key, x0 + h * u) - L(key, x0 - h * u)) / (2 * h)
            ana = float((bwd[gkey] * u).sum())
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (key, num, ana)


def test_projection_layer_backward_finite_differences():
    """The layer with its in/out projections: directional central differences
    for the hidden states and every projection weight, against the composed
    backward (the core's own gradients are pinned above)."""
    w = gi.Workload("fdp", 10, 1, 2, 4, "fp32", seq="varlen", init_state=True, final_state=True,
                    seed=6)
    inp = gi.make_inputs(w, seqlens=[7, 3], A_range=(0.05, 0.5))
    hk, hv, d, sc, H = 1, 2, 4, 0.5, 6
    rng = np.random.default_rng(9)
    T, C = 10, w.channels
    X = rng.standard_normal((T, H))
    W = {"x": rng.standard_normal((C, H)) / np.sqrt(H), "z": rng.standard_normal((hv * d, H)) / np.sqrt(H),
         "a": rng.standard_normal((hv, H)) / np.sqrt(H), "b": rng.standard_normal((hv, H)) / np.sqrt(H),
         "out": rng.standard_normal((H, hv * d)) / np.sqrt(hv * d)}
    params = {k: inp[k].astype(np.float64) for k in ("w_conv", "A_log", "dt_bias", "w_norm")}
    S0 = inp["S0"].astype(np.float64)
    dY = rng.standard_normal((T, H))
    dST = inp["dS_T"].astype(np.float64)
    cu = inp["cu_seqlens"]
    fwd = oracle.proj_layer_fwd(X, W, params, cu, hk, hv, d, sc, S0=S0)
    bwd = oracle.proj_layer_bwd(X, W, fwd, dY, hk, hv, d, sc, dS_T=dST)

    def L(X_, W_):
        f = oracle.proj_layer_fwd(X_, W_, params, cu, hk, hv, d, sc, S0=S0)
        return float((f["Y"] * dY).sum() + (f["S_final"] * dST).sum())

    h = 1e-6
    for _ in range(2):
        u = rng.standard_normal(X.shape)
        num = (L(X + h * u, W) - L(X - h * u, W)) / (2 * h)
        ana = float((bwd["dX"] * u).sum())
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), ("X", num, ana)
    for key in W:
        u = rng.standard_normal(W[key].shape)
        Wp, Wm = dict(W), dict(W)
        Wp[key], Wm[key] = W[key] + h * u, W[key] - h * u
        num = (L(X, Wp) - L(X, Wm)) / (2 * h)
        ana = float((bwd["dW"][key] * u).sum())
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (key, num, ana)
