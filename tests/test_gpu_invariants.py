"""The gated delta rule's invariants, checked on the GPU through the C ABI,
in both chunk flows (the composite gdn_chunk_fwd / gdn_chunk_bwd, and the
training flow that saves the chunk states: gdn_chunk_prepare_bwd,
gdn_chunk_fwd_states_save, gdn_chunk_bwd_reverse, gdn_chunk_bwd_grads),
each on inputs built for it.  The same
invariants pin the oracle on the CPU; here they probe regimes that random
inputs do not reach: no write and no decay, exact recall, overwrite,
infinite decay, continuation across calls, grouped values.

The recurrence: S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t (scale q_t), S [d_v][d_k] per (sequence, value head)."""
import numpy as np
import pytest
import torch

from gated_deltanet_layer_causal_amd import capi as L
from gated_deltanet_layer_causal_amd import inputs as gi
from tests.gpu_util import DEV, FWD_TOL_BF16, GRAD_TOL_BF16, TOL_FP32, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _run(q, k, v, g, beta, lens, scale, S0=None, dtype="bf16", dout=None, dS_final=None, seg=0,
         flow="composite"):
    """q, k [T, hk, d]; v [T, hv, d]; g, beta [T, hv] (float arrays, bf16-exact
    for bf16).  Returns o, S_final (and dq, dk, dv, dg, dbeta, dS0 if dout).
    seg > 0 runs the segment-parallel state scan with segments of seg chunks."""
    T, hk, d = q.shape
    hv = v.shape[1]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cu = gi.cu_from_lengths(lens)
    N = len(lens)
    sh = L.make_shape(N, T, hk, hv, d, L.GDN_BF16 if dtype == "bf16" else L.GDN_FP32, seg)
    y = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    yt = dev(y, tdt)
    C = hk * d
    qt, kt, vt = yt[:, :C], yt[:, C:2 * C], yt[:, 2 * C:]
    gt, bt = dev(g), dev(beta)
    cut = torch.from_numpy(cu).to(DEV)
    S0t = dev(S0) if S0 is not None else None
    Sf = torch.empty((N, hv, d, d), dtype=torch.float32, device=DEV)
    o = torch.empty((T, hv, d), dtype=tdt, device=DEV)
    ws = torch.empty(max(L.gdn_chunk_fwd_workspace(sh), L.gdn_chunk_bwd_workspace(sh)),
                     dtype=torch.uint8, device=DEV)
    if flow == "composite":
        L.gdn_chunk_fwd(sh, qt, kt, vt, gt, bt, scale, S0t, Sf, cut, o, ws)
    else:
        L.gdn_chunk_prepare_bwd(sh, qt, kt, gt, bt, scale, cut, ws)
        L.gdn_chunk_fwd_states_save(sh, qt, kt, vt, scale, S0t, Sf, cut, o, ws)
    out = {"o": host(o), "S_final": host(Sf)}
    if dout is not None:
        dy = torch.empty_like(yt)
        dq, dk, dv = dy[:, :C], dy[:, C:2 * C], dy[:, 2 * C:]
        dg, db = torch.empty_like(gt), torch.empty_like(bt)
        dS0 = torch.empty_like(Sf)
        dot = dev(dout, tdt)
        dSft = dev(dS_final) if dS_final is not None else None
        if flow == "composite":
            L.gdn_chunk_bwd(sh, qt, kt, vt, gt, bt, scale, S0t, cut, dot, dSft, dq, dk, dv, dg, db,
                            dS0, ws)
        else:
            L.gdn_chunk_bwd_reverse(sh, qt, kt, scale, cut, dot, dSft, dv, dS0, ws)
            L.gdn_chunk_bwd_grads(sh, qt, kt, bt, scale, cut, dot, dv, dq, dk, dg, db, ws)
        out.update(dq=host(dq).reshape(T, hk, d), dk=host(dk).reshape(T, hk, d),
                   dv=host(dv).reshape(T, hv, d), dg=host(dg), dbeta=host(db), dS0=host(dS0))
    torch.cuda.synchronize()
    return out


def _unit(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _rb(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return gi.round_bf16(a) if dtype == "bf16" else a


def _tol(dtype, grad=False):
    return TOL_FP32 if dtype == "fp32" else (GRAD_TOL_BF16 if grad else FWD_TOL_BF16)


CASES = [("fp32", 1, 2, 32, [64, 37]), ("bf16", 2, 4, 128, [150, 70])]


@pytest.mark.parametrize("dtype,hk,hv,d,lens", CASES, ids=["fp32", "bf16"])
@pytest.mark.parametrize("seg", [0, 1], ids=["seq", "seg1"])
@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_I1_no_write_no_decay_keeps_state(dtype, hk, hv, d, lens, seg, flow):
    """beta = 0 and g = 0: the state stays S0 (exactly: no term is added and
    the decay is 1) and o_t = S0 (scale q_t)."""
    rng = np.random.default_rng(21)
    T, G = sum(lens), hv // hk
    q = _rb(_unit(rng.standard_normal((T, hk, d))), dtype)
    k = _rb(_unit(rng.standard_normal((T, hk, d))), dtype)
    v = _rb(rng.standard_normal((T, hv, d)), dtype)
    z = np.zeros((T, hv), np.float32)
    S0 = (0.3 * rng.standard_normal((len(lens), hv, d, d))).astype(np.float32)
    sc = d ** -0.5
    r = _run(q, k, v, z, z, lens, sc, S0, dtype, seg=seg, flow=flow)
    np.testing.assert_array_equal(r["S_final"], S0.astype(np.float64))
    cu = gi.cu_from_lengths(lens)
    ref = np.zeros((T, hv, d))
    for n in range(len(lens)):
        for t in range(cu[n], cu[n + 1]):
            for h in range(hv):
                ref[t, h] = S0[n, h].astype(np.float64) @ (sc * q[t, h // G].astype(np.float64))
    assert_close("o", r["o"], ref, _tol(dtype))


@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_I2_exact_recall_with_orthonormal_keys(flow):
    """beta = 1, g = 0, S0 = 0 and orthonormal keys (T <= d_k): the final state
    maps each key to its value, S_T k_j = v_j."""
    rng = np.random.default_rng(22)
    d, T = 32, 32
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[:T].reshape(T, 1, d).astype(np.float32)      # rows orthonormal
    v = rng.standard_normal((T, 2, d)).astype(np.float32)
    q = _unit(rng.standard_normal((T, 1, d))).astype(np.float32)
    one, zero = np.ones((T, 2), np.float32), np.zeros((T, 2), np.float32)
    r = _run(q, k, v, zero, one, [T], 1.0, None, "fp32", flow=flow)
    for h in range(2):
        recall = r["S_final"][0, h] @ k[:, 0].T.astype(np.float64)      # [d_v, T]
        assert_close(f"recall h{h}", recall.T, v[:, h].astype(np.float64), TOL_FP32)


@pytest.mark.parametrize("dtype,hk,hv,d,lens", CASES, ids=["fp32", "bf16"])
@pytest.mark.parametrize("seg", [0, 1], ids=["seq", "seg1"])
@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_I3_unit_key_full_write_overwrites(dtype, hk, hv, d, lens, seg, flow):
    """Unit k_t and beta_t = 1: S_t k_t = v_t whatever g_t and S_{t-1}; so the
    final state maps each sequence's last key to its last value."""
    rng = np.random.default_rng(23)
    T, G = sum(lens), hv // hk
    q = _rb(_unit(rng.standard_normal((T, hk, d))), dtype)
    k = _unit(rng.standard_normal((T, hk, d)))
    k = _rb(k, dtype)
    v = _rb(rng.standard_normal((T, hv, d)), dtype)
    g = -rng.uniform(0.0, 0.5, (T, hv)).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((len(lens), hv, d, d))).astype(np.float32)
    r = _run(q, k, v, g, np.ones((T, hv), np.float32), lens, d ** -0.5, S0, dtype, seg=seg)
    cu = gi.cu_from_lengths(lens)
    for n in range(len(lens)):
        t = cu[n + 1] - 1
        for h in range(hv):
            kk = k[t, h // G].astype(np.float64)
            # the bf16 key is unit only up to its rounding: S_t k_t = v_t + (1 - |k|^2) (...)
            got = r["S_final"][n, h] @ kk / (kk @ kk)
            assert_close(f"S k = v (seq {n}, head {h})", got, v[t, h].astype(np.float64),
                         _tol(dtype))


@pytest.mark.parametrize("dtype,hk,hv,d,lens", CASES, ids=["fp32", "bf16"])
@pytest.mark.parametrize("seg", [0, 1], ids=["seq", "seg1"])
@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_I4_infinite_decay_is_local(dtype, hk, hv, d, lens, seg, flow):
    """g -> -infinity (the decay underflows to zero): nothing of the past
    reaches token t, o_t = beta_t (k_t . scale q_t) v_t, and the final state is
    the last write."""
    rng = np.random.default_rng(24)
    T, G = sum(lens), hv // hk
    q = _rb(_unit(rng.standard_normal((T, hk, d))), dtype)
    k = _rb(_unit(rng.standard_normal((T, hk, d))), dtype)
    v = _rb(rng.standard_normal((T, hv, d)), dtype)
    g = np.full((T, hv), -200.0, np.float32)
    beta = rng.uniform(0.1, 0.9, (T, hv)).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((len(lens), hv, d, d))).astype(np.float32)
    sc = d ** -0.5
    r = _run(q, k, v, g, beta, lens, sc, S0, dtype, seg=seg, flow=flow)
    q64, k64, v64, b64 = (a.astype(np.float64) for a in (q, k, v, beta))
    ref = np.zeros((T, hv, d))
    for h in range(hv):
        kq = np.sum(k64[:, h // G] * sc * q64[:, h // G], axis=-1)
        ref[:, h] = (b64[:, h] * kq)[:, None] * v64[:, h]
    assert_close("o", r["o"], ref, _tol(dtype))
    cu = gi.cu_from_lengths(lens)
    for n in range(len(lens)):
        t = cu[n + 1] - 1
        for h in range(hv):
            last = b64[t, h] * np.outer(v64[t, h], k64[t, h // G])
            assert_close(f"S_final (seq {n}, head {h})", r["S_final"][n, h], last, _tol(dtype))


@pytest.mark.parametrize("seg", [0, 1], ids=["seq", "seg1"])
@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_I6_continuation_through_the_final_state(seg, flow):
    """Splitting a sequence inside a chunk and feeding the first part's final
    state in as the second part's initial state reproduces o and S_final
    (also with the segmented scan, whose segments are then a third way of
    cutting the same sequence)."""
    rng = np.random.default_rng(26)
    hk, hv, d, T, cut = 2, 4, 128, 300, 130
    q = _rb(_unit(rng.standard_normal((T, hk, d))), "bf16")
    k = _rb(_unit(rng.standard_normal((T, hk, d))), "bf16")
    v = _rb(rng.standard_normal((T, hv, d)), "bf16")
    g = -rng.uniform(0.0, 0.3, (T, hv)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (T, hv)).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((1, hv, d, d))).astype(np.float32)
    sc = d ** -0.5
    whole = _run(q, k, v, g, beta, [T], sc, S0, flow=flow)
    a = _run(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], [cut], sc, S0, seg=seg, flow=flow)
    b = _run(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], [T - cut], sc,
             a["S_final"].astype(np.float32), seg=seg, flow=flow)
    assert_close("o", np.concatenate([a["o"], b["o"]]), whole["o"], FWD_TOL_BF16)
    assert_close("S_final", b["S_final"], whole["S_final"], FWD_TOL_BF16)


@pytest.mark.parametrize("seg", [0, 1], ids=["seq", "seg1"])
@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_I7_grouped_values_equal_repeated_keys(seg, flow):
    """Grouped values (2 key heads for 4 value heads) equal explicitly
    repeated q and k (4 key heads), forward and backward, with dq and dk of
    the grouped run the sums over each group."""
    rng = np.random.default_rng(27)
    hk, hv, d, lens = 2, 4, 128, [150, 70]
    T, G = sum(lens), hv // hk
    q = _rb(_unit(rng.standard_normal((T, hk, d))), "bf16")
    k = _rb(_unit(rng.standard_normal((T, hk, d))), "bf16")
    v = _rb(rng.standard_normal((T, hv, d)), "bf16")
    g = -rng.uniform(0.0, 0.3, (T, hv)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (T, hv)).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((len(lens), hv, d, d))).astype(np.float32)
    dout = _rb(rng.standard_normal((T, hv, d)), "bf16")
    dSf = rng.standard_normal((len(lens), hv, d, d)).astype(np.float32)
    sc = d ** -0.5
    grp = _run(q, k, v, g, beta, lens, sc, S0, dout=dout, dS_final=dSf, seg=seg, flow=flow)
    rep = _run(np.repeat(q, G, axis=1), np.repeat(k, G, axis=1), v, g, beta, lens, sc, S0,
               dout=dout, dS_final=dSf, flow=flow)
    for key in ("o", "S_final"):
        assert_close(key, grp[key], rep[key], FWD_TOL_BF16)
    for key in ("dv", "dg", "dbeta", "dS0"):
        assert_close(key, grp[key], rep[key], GRAD_TOL_BF16)
    for key in ("dq", "dk"):
        summed = rep[key].reshape(T, hk, G, d).sum(axis=2)
        assert_close(key, grp[key], summed, GRAD_TOL_BF16)
