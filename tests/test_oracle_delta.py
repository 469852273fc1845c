"""Pins for the oracle's gated delta rule (CPU only).

Each check ties the oracle to something other than itself: exact values
worked by hand, brute-force unrolled matrix products, closed-form special
cases, the chunked WY/UT form, finite differences and the adjoint identity.
"""
import os

import numpy as np
import pytest

import oracle
from tests.chunked_model import chunked_bwd, chunked_fwd

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, T, Hk, Hv, d, lens=None, S0=False, mild=True, unit=True):
    lens = [T] if lens is None else lens
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, Hk, d))
    k = rng.standard_normal((T, Hk, d))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, d))
    g = -rng.uniform(0.0, 0.3 if mild else 8.0, (T, Hv))
    beta = rng.uniform(0.05, 0.95, (T, Hv))
    s0 = 0.3 * rng.standard_normal((len(lens), Hv, d, d)) if S0 else None
    return q, k, v, g, beta, cu, s0


# ------------------------------------------------------------------ golden
def test_hand_worked_three_tokens():
    rows, S_ref = [], None
    for line in open(os.path.join(GOLD, "delta_hand_3tok.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("S"):
            S_ref = np.array([float(x) for x in line.split()[1:]]).reshape(2, 2)
        else:
            rows.append([float(x) for x in line.split()])
    rows = np.array(rows)
    T = len(rows)
    k = rows[:, 1:3].reshape(T, 1, 2)
    v = rows[:, 3:5].reshape(T, 1, 2)
    beta = rows[:, 5:6]
    g = np.log(rows[:, 6:7])
    q = rows[:, 7:9].reshape(T, 1, 2)
    o_ref = rows[:, 9:11]
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, [0, T], 1.0)
    np.testing.assert_allclose(o[:, 0], o_ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Sf[0, 0], S_ref, rtol=0, atol=1e-15)
    o2, _ = oracle.delta_fwd(q, k, v, g, beta, [0, T], 0.5)
    np.testing.assert_allclose(o2[:, 0], 0.5 * o_ref, rtol=0, atol=1e-15)


# ------------------------------------------------------------------ V1 brute force
def _brute(q, k, v, g, beta, cu, scale, S0):
    """S_t = S_0 P_1...P_t + sum_s beta_s v_s k_s^T P_{s+1}...P_t,
    P_i = exp(g_i) (I - beta_i k_i k_i^T), built as explicit matrices."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    G = Hv // Hk
    o = np.zeros((T, Hv, dv))
    Sf = np.zeros((len(cu) - 1, Hv, dv, dk))
    for n in range(len(cu) - 1):
        for h in range(Hv):
            kh = h // G
            t0, t1 = cu[n], cu[n + 1]
            Pm = [np.exp(g[t, h]) * (np.eye(dk) - beta[t, h] * np.outer(k[t, kh], k[t, kh]))
                  for t in range(t0, t1)]
            base = np.zeros((dv, dk)) if S0 is None else S0[n, h]
            for t in range(t0, t1):
                prod = np.eye(dk)
                for i in range(t0, t + 1):
                    prod = prod @ Pm[i - t0]
                St = base @ prod
                for s in range(t0, t + 1):
                    tail = np.eye(dk)
                    for i in range(s + 1, t + 1):
                        tail = tail @ Pm[i - t0]
                    St = St + beta[s, h] * np.outer(v[s, h], k[s, kh]) @ tail
                o[t, h] = St @ (scale * q[t, kh])
                if t == t1 - 1:
                    Sf[n, h] = St
    return o, Sf


@pytest.mark.parametrize("lens,Hk,Hv,d,S0", [([9], 1, 1, 4, False), ([5, 7], 1, 2, 3, True),
                                             ([3, 1, 6], 2, 4, 5, True)])
def test_brute_force_unrolled_products(lens, Hk, Hv, d, S0):
    rng = np.random.default_rng(11)
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), Hk, Hv, d, lens, S0, unit=False)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.7, s0)
    ob, Sb = _brute(q, k, v, g, beta, cu, 0.7, s0)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sf, Sb, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ invariants
def test_I1_no_write_no_decay_keeps_state():
    rng = np.random.default_rng(1)
    q, k, v, g, beta, cu, s0 = _rand_case(rng, 20, 1, 2, 6, [20], True)
    g[:] = 0.0
    beta[:] = 0.0
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.5, s0)
    np.testing.assert_allclose(Sf, s0, rtol=0, atol=1e-15)
    ref = np.einsum("hij,thj->thi", s0[0], 0.5 * q[:, [0, 0]])
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)


def test_I2_exact_recall_orthonormal_keys():
    rng = np.random.default_rng(2)
    d = 8
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T.reshape(d, 1, d)            # rows are orthonormal keys
    v = rng.standard_normal((d, 1, d))
    g = np.zeros((d, 1))
    beta = np.ones((d, 1))
    q = k.copy()
    _, Sf = oracle.delta_fwd(q, k, v, g, beta, [0, d], 1.0)
    # querying the final state with k_j returns v_j exactly
    rec = np.einsum("ij,tj->ti", Sf[0, 0], k[:, 0])
    np.testing.assert_allclose(rec, v[:, 0], rtol=0, atol=1e-12)


def test_I3_delta_rule_overwrites_with_unit_key():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, cu, s0 = _rand_case(rng, 12, 1, 1, 5, [12], True, mild=False)
    beta[:] = 1.0
    for t_end in (1, 5, 12):
        _, Sf = oracle.delta_fwd(q[:t_end], k[:t_end], v[:t_end], g[:t_end], beta[:t_end],
                                 [0, t_end], 1.0, s0)
        np.testing.assert_allclose(Sf[0, 0] @ k[t_end - 1, 0], v[t_end - 1, 0], atol=1e-12)


def test_I4_infinite_decay_is_local():
    rng = np.random.default_rng(4)
    q, k, v, g, beta, cu, s0 = _rand_case(rng, 10, 1, 2, 4, [10], True)
    g[:] = -1e4      # exp(g) == 0 in double
    o, _ = oracle.delta_fwd(q, k, v, g, beta, cu, 0.9, s0)
    kq = np.einsum("tj,tj->t", k[:, 0], 0.9 * q[:, 0])
    ref = beta[:, :, None] * kq[:, None, None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)


def test_I5_varlen_equals_separate_runs():
    rng = np.random.default_rng(5)
    lens = [7, 1, 13, 4]
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), 2, 4, 6, lens, True)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.6, s0)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, Sn = oracle.delta_fwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a], 0.6,
                                  s0[n:n + 1])
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(Sf[n], Sn[0])


def test_empty_sequences_pass_state_through():
    """A sequence without tokens applies no step of the recurrence: its final
    state is its initial state and the gradient of its initial state is the
    final state's gradient; the other sequences are the same as without it."""
    rng = np.random.default_rng(15)
    lens = [0, 9, 0, 6, 0]
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), 1, 2, 5, lens, True)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.6, s0)
    dout = rng.standard_normal(o.shape)
    dST = rng.standard_normal(Sf.shape)
    *_, dS0 = oracle.delta_bwd(q, k, v, g, beta, cu, 0.6, dout, s0, dST)
    keep = [n for n, ln in enumerate(lens) if ln > 0]
    cu2 = np.concatenate([[0], np.cumsum([lens[n] for n in keep])]).astype(np.int32)
    o2, Sf2 = oracle.delta_fwd(q, k, v, g, beta, cu2, 0.6, s0[keep])
    for n, ln in enumerate(lens):
        if ln == 0:
            np.testing.assert_array_equal(Sf[n], s0[n])
            np.testing.assert_array_equal(dS0[n], dST[n])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(Sf[keep], Sf2)


def test_I6_continuation_through_final_state():
    rng = np.random.default_rng(6)
    q, k, v, g, beta, cu, s0 = _rand_case(rng, 30, 1, 2, 5, [30], True)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.6, s0)
    o1, S1 = oracle.delta_fwd(q[:11], k[:11], v[:11], g[:11], beta[:11], [0, 11], 0.6, s0)
    o2, S2 = oracle.delta_fwd(q[11:], k[11:], v[11:], g[11:], beta[11:], [0, 19], 0.6, S1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S2, Sf, rtol=1e-13, atol=1e-14)


def test_I7_grouped_values_equal_repeated_keys():
    """Native grouped-value heads equal explicitly repeated q/k (miles page, GB300
    results: native GVA vs repeated q/k), with dq/dk summed over each group."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, cu, s0 = _rand_case(rng, 17, 2, 6, 4, [9, 8], True)
    dout = rng.standard_normal(v.shape)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.5, s0)
    qr, kr = np.repeat(q, 3, axis=1), np.repeat(k, 3, axis=1)
    o2, Sf2 = oracle.delta_fwd(qr, kr, v, g, beta, cu, 0.5, s0)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-15)
    g1 = oracle.delta_bwd(q, k, v, g, beta, cu, 0.5, dout, s0)
    g2 = oracle.delta_bwd(qr, kr, v, g, beta, cu, 0.5, dout, s0)
    T = q.shape[0]
    np.testing.assert_allclose(g1[0], g2[0].reshape(T, 2, 3, 4).sum(2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g1[1], g2[1].reshape(T, 2, 3, 4).sum(2), rtol=1e-12, atol=1e-13)
    for a, b in zip(g1[2:], g2[2:]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ V2 chunked == sequential
@pytest.mark.parametrize("C", [4, 8, 16])
@pytest.mark.parametrize("mild", [True, False])
def test_chunked_form_equals_sequential(C, mild):
    rng = np.random.default_rng(20 + C)
    lens = [21, 3, 16, 10]
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), 2, 4, 6, lens, True, mild=mild)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.4, s0)
    oc, Sc = chunked_fwd(q, k, v, g, beta, cu, 0.4, s0, C=C)
    np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sc, Sf, rtol=1e-11, atol=1e-12)
    dout = rng.standard_normal(v.shape)
    dSf = rng.standard_normal(Sf.shape)
    ref = oracle.delta_bwd(q, k, v, g, beta, cu, 0.4, dout, s0, dSf)
    got = chunked_bwd(q, k, v, g, beta, cu, 0.4, dout, s0, dSf, C=C)
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-10, err_msg=name)


# ------------------------------------------------------------------ V3 finite differences
def _fd_dir(f, x, u, h=1e-6):
    return (f(x + h * u) - f(x - h * u)) / (2 * h)


def test_delta_backward_matches_finite_differences():
    rng = np.random.default_rng(8)
    lens = [6, 5]
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), 1, 2, 3, lens, True, unit=False)
    dout = rng.standard_normal(v.shape)
    dSf = rng.standard_normal(s0.shape)
    sc = 0.8
    dq, dk, dv, dg, dbeta, dS0 = oracle.delta_bwd(q, k, v, g, beta, cu, sc, dout, s0, dSf)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0)

    def loss(**kw):
        a = dict(args)
        a.update(kw)
        o, Sf = oracle.delta_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], cu, sc, a["s0"])
        return float((o * dout).sum() + (Sf * dSf).sum())

    grads = dict(q=dq, k=dk, v=dv, g=dg, beta=dbeta, s0=dS0)
    for name, gr in grads.items():
        x0 = args[name]
        # element-wise central differences over every entry
        num = np.zeros_like(x0)
        it = np.nditer(x0, flags=["multi_index"])
        for _ in it:
            e = np.zeros_like(x0)
            e[it.multi_index] = 1.0
            num[it.multi_index] = _fd_dir(lambda x: loss(**{name: x}), x0, e)
        np.testing.assert_allclose(gr, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_adjoint_identity():
    """For fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear, so
    <do, o> + <dS_T, S_T> = <dv, v> + <dS0, S0>."""
    rng = np.random.default_rng(9)
    lens = [40, 25]
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), 2, 4, 8, lens, True)
    dout = rng.standard_normal(v.shape)
    dSf = rng.standard_normal(s0.shape)
    o, Sf = oracle.delta_fwd(q, k, v, g, beta, cu, 0.3, s0)
    _, _, dv, _, _, dS0 = oracle.delta_bwd(q, k, v, g, beta, cu, 0.3, dout, s0, dSf)
    lhs = (dout * o).sum() + (dSf * Sf).sum()
    rhs = (dv * v).sum() + (dS0 * s0).sum()
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


def test_long_sequence_checkpoint_segments():
    """Backward across several 64-token checkpoint segments (ragged tail)
    equals the chunked form at chunk 64 and 32."""
    rng = np.random.default_rng(10)
    lens = [150, 64, 1]
    q, k, v, g, beta, cu, s0 = _rand_case(rng, sum(lens), 1, 2, 4, lens, True)
    dout = rng.standard_normal(v.shape)
    ref = oracle.delta_bwd(q, k, v, g, beta, cu, 0.5, dout, s0)
    for C in (64, 32):
        got = chunked_bwd(q, k, v, g, beta, cu, 0.5, dout, s0, None, C=C)
        for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
            np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-10, err_msg=name)


@pytest.mark.parametrize("seg", [1, 2, 3])
def test_segmented_scan_equals_sequential(seg):
    """The segment-parallel scan's algebra (segment summaries B, Phi and dB,
    then S_{s+1} = S_s Phi_s + B_s forward and dS_{s-1} = dS_s Phi_s^T + dB_s
    backward) reproduces the oracle's S_final and dS0 and the sequential
    states and state gradients at every segment boundary, with mild decay so
    that the state crosses segments, several sequences and ragged tails."""
    from tests.chunked_model import _chunks, _rev_dS, _run_chunks, segmented_scan
    rng = np.random.default_rng(40 + seg)
    hk, hv, d, C = 1, 2, 8, 4
    lens = [23, 1, 9, 0, 17]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, hk, d))
    k = rng.standard_normal((T, hk, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, hv, d))
    g = -rng.uniform(0.0, 0.2, (T, hv))
    beta = rng.uniform(0.2, 0.9, (T, hv))
    S0 = rng.standard_normal((len(lens), hv, d, d))
    dSf = rng.standard_normal((len(lens), hv, d, d))
    dout = rng.standard_normal((T, hv, d))
    sc = 0.5
    starts, Sf, ends, dS0 = segmented_scan(q, k, v, g, beta, cu, sc, dout, S0, dSf, C=C, seg=seg)
    _, Sf_ref = oracle.delta_fwd(q, k, v, g, beta, cu, sc, S0)
    ref = oracle.delta_bwd(q, k, v, g, beta, cu, sc, dout, S0, dSf)
    np.testing.assert_allclose(Sf, Sf_ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dS0, ref[5], rtol=1e-10, atol=1e-10)
    for n in range(len(lens)):
        chunks = _chunks(cu[n], cu[n + 1], C)
        for h in range(hv):
            Q, K, V = sc * q[:, 0], k[:, 0], v[:, h]
            for s in range(len(starts[n, h])):
                before = chunks[: s * seg]
                S = _run_chunks(before, Q, K, V, g[:, h], beta[:, h], S0[n, h])
                np.testing.assert_allclose(starts[n, h][s], S, rtol=1e-10, atol=1e-10)
                after = chunks[(s + 1) * seg:]
                dS = _rev_dS(after, Q, K, V, g[:, h], beta[:, h], dout[:, h], dSf[n, h])
                np.testing.assert_allclose(ends[n, h][s], dS, rtol=1e-10, atol=1e-10)
