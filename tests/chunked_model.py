"""Chunked (WY/UT-transform) form of the gated delta rule, in float64 numpy.

Test helper only.  It is an independent, blocked restatement of the
recurrence that the GPU kernels implement, used to show on the CPU that
"chunked equals sequential" (against the token-by-token oracle) for the
forward and the backward, before any kernel runs.

Per chunk of L tokens with start state S (d_v x d_k):
    gam = inclusive cumsum of g inside the chunk,  Gam = exp(gam)
    D[t,s] = exp(gam_t - gam_s) for s <= t
    A = strictly-lower( beta_t D[t,s] k_t.k_s ),   Tinv = (I + A)^-1
    M = Tinv diag(beta)
    R = V - diag(Gam) K S^T          Delta = M R
    P = lower( D * (scale Q) K^T )
    O = diag(Gam) (scale Q) S^T + P Delta
    S' = Gam_L S + (diag(dec) Delta)^T K,  dec_t = exp(gam_L - gam_t)
"""
from __future__ import annotations

import numpy as np


def _chunk_fwd(Q, K, V, gg, bb, S):
    L = Q.shape[0]
    gam = np.cumsum(gg)
    Gam = np.exp(gam)
    diff = gam[:, None] - gam[None, :]
    low = np.tril(np.ones((L, L), dtype=bool))
    D = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
    KK = K @ K.T
    A = np.tril(bb[:, None] * D * KK, -1)
    Tinv = np.linalg.inv(np.eye(L) + A)
    M = Tinv * bb[None, :]
    R = V - Gam[:, None] * (K @ S.T)
    Dl = M @ R
    P = D * (Q @ K.T)
    O = Gam[:, None] * (Q @ S.T) + P @ Dl
    dec = np.exp(gam[-1] - gam)
    Snew = Gam[-1] * S + (dec[:, None] * Dl).T @ K
    cache = dict(gam=gam, Gam=Gam, D=D, KK=KK, A=A, Tinv=Tinv, M=M, R=R, Dl=Dl, P=P, dec=dec)
    return O, Snew, cache


def chunked_fwd(q, k, v, g, beta, cu, scale, S0=None, C=64):
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    G = Hv // Hk
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    Sf = np.zeros((N, Hv, dv, dk))
    for n in range(N):
        for h in range(Hv):
            kh = h // G
            S = np.zeros((dv, dk)) if S0 is None else S0[n, h].astype(np.float64).copy()
            for c0 in range(cu[n], cu[n + 1], C):
                c1 = min(c0 + C, cu[n + 1])
                O, S, _ = _chunk_fwd(scale * q[c0:c1, kh], k[c0:c1, kh], v[c0:c1, h],
                                     g[c0:c1, h], beta[c0:c1, h], S)
                o[c0:c1, h] = O
            Sf[n, h] = S
    return o, Sf


def chunked_bwd(q, k, v, g, beta, cu, scale, dout, S0=None, dS_final=None, C=64):
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    G = Hv // Hk
    N = len(cu) - 1
    dq = np.zeros_like(q, dtype=np.float64)
    dkk = np.zeros_like(k, dtype=np.float64)
    dvv = np.zeros((T, Hv, dv))
    dg = np.zeros((T, Hv))
    dbeta = np.zeros((T, Hv))
    dS0 = np.zeros((N, Hv, dv, dk))
    for n in range(N):
        for h in range(Hv):
            kh = h // G
            starts = list(range(cu[n], cu[n + 1], C))
            S = np.zeros((dv, dk)) if S0 is None else S0[n, h].astype(np.float64).copy()
            states = []
            for c0 in starts:                       # forward: chunk-start states
                c1 = min(c0 + C, cu[n + 1])
                states.append(S)
                _, S, _ = _chunk_fwd(scale * q[c0:c1, kh], k[c0:c1, kh], v[c0:c1, h],
                                     g[c0:c1, h], beta[c0:c1, h], S)
            dS = np.zeros((dv, dk)) if dS_final is None else dS_final[n, h].astype(np.float64).copy()
            for ci in reversed(range(len(starts))):
                c0 = starts[ci]
                c1 = min(c0 + C, cu[n + 1])
                S = states[ci]
                Q = scale * q[c0:c1, kh]
                K = k[c0:c1, kh]
                bb = beta[c0:c1, h]
                dO = dout[c0:c1, h]
                _, _, c = _chunk_fwd(Q, K, v[c0:c1, h], g[c0:c1, h], bb, S)
                Gam, D, A, Tinv, M, R, Dl, P, dec = (c[x] for x in
                                                     ("Gam", "D", "A", "Tinv", "M", "R", "Dl", "P", "dec"))
                L = c1 - c0
                dSp = dS
                # sequential part
                dDl = P.T @ dO + dec[:, None] * (K @ dSp.T)
                dR = M.T @ dDl
                dS = Gam[-1] * dSp + dO.T @ (Gam[:, None] * Q) - (Gam[:, None] * dR).T @ K
                # chunk-parallel part
                dM = dDl @ R.T
                dP = np.tril(dO @ Dl.T)
                dTinv = np.tril(dM * bb[None, :], -1)
                dA = np.tril(-(Tinv.T @ dTinv @ Tinv.T), -1)
                dbe = (dM * Tinv).sum(axis=0) + (dA * D * c["KK"]).sum(axis=1)
                dQ = Gam[:, None] * (dO @ S) + (dP * D) @ K
                WA = dA * bb[:, None] * D
                dK = ((dP * D).T @ Q - Gam[:, None] * (dR @ S) + dec[:, None] * (Dl @ dSp)
                      + WA @ K + WA.T @ K)
                # dg_i = sum_{t >= i} dgam_t, assembled from three parts whose
                # terms all carry the decay across token i:
                # chunk-start terms y_t (and the state term on the last token)
                # as a suffix sum
                y = ((dO * (Gam[:, None] * (Q @ S.T))).sum(axis=1)
                     - (dR * (Gam[:, None] * (K @ S.T))).sum(axis=1))
                y[-1] += Gam[-1] * (dSp * S).sum()
                # pair terms E[t, s] (s < t) add to dgam_t and subtract from
                # dgam_s: their part of dg_i is the box sum over t >= i > s
                # (the diagonal of dP o P would cancel exactly: left out)
                E = np.tril(dP * P, -1) + dA * A
                colsuf = np.cumsum(E[::-1], axis=0)[::-1]       # sum over rows >= t
                box = np.array([colsuf[i, :i].sum() for i in range(L)])
                # dec_t = exp(gam_L - gam_t): its gradient puts -z_t on token t
                # and +sum(z) on the last token; in dg that is the exclusive
                # prefix sum of z
                z = dec * ((Dl @ dSp) * K).sum(axis=1)
                dg[c0:c1, h] = box + np.cumsum(y[::-1])[::-1] + (np.cumsum(z) - z)
                dbeta[c0:c1, h] = dbe
                dvv[c0:c1, h] = dR
                dq[c0:c1, kh] += scale * dQ
                dkk[c0:c1, kh] += dK
            dS0[n, h] = dS
    return dq, dkk, dvv, dg, dbeta, dS0


# ---------------------------------------------------------------------------
# Segment-parallel form of the state recurrences.  Over the chunks of one
# segment the state map is affine, S_end = S_start Phi + B: B is the end state
# reached from a zero start, Phi = A_1 ... A_L (A_c the chunk's map of the
# state with no values) is reached by running the same chunks from identity
# rows with zero values.  The state gradient maps through the transposes:
# dS_start = dS_end Phi^T + dB, dB the start gradient reached from a zero
# end gradient.

def _chunks(c_lo, c_hi, C):
    return [(c0, min(c0 + C, c_hi)) for c0 in range(c_lo, c_hi, C)]


def _run_chunks(spans, Q, K, V, gg, bb, S):
    for c0, c1 in spans:
        _, S, _ = _chunk_fwd(Q[c0:c1], K[c0:c1], V[c0:c1], gg[c0:c1], bb[c0:c1], S)
    return S


def _rev_dS(spans, Q, K, V, gg, bb, dO, dSp):
    """The reverse recurrence of the state gradient over `spans` (last chunk
    first) from dSp at their end; returns the gradient at their start.  It
    does not depend on the states."""
    for c0, c1 in reversed(spans):
        L = c1 - c0
        _, _, c = _chunk_fwd(Q[c0:c1], K[c0:c1], np.zeros((L, dSp.shape[0])), gg[c0:c1],
                             bb[c0:c1], np.zeros_like(dSp))
        Gam, M, P, dec = c["Gam"], c["M"], c["P"], c["dec"]
        dDl = P.T @ dO[c0:c1] + dec[:, None] * (K[c0:c1] @ dSp.T)
        dR = M.T @ dDl
        dSp = Gam[-1] * dSp + dO[c0:c1].T @ (Gam[:, None] * Q[c0:c1]) - (Gam[:, None] * dR).T @ K[c0:c1]
    return dSp


def segmented_scan(q, k, v, g, beta, cu, scale, dout, S0=None, dS_final=None, C=64, seg=2):
    """Per (sequence, value head): the segment start states, S_final, the
    state gradients at the segment ends and dS0, by the segmented scan
    (summaries per segment, then the combines).  Returns
    (starts, S_final, dS_ends, dS0), starts / dS_ends as {(n, h): [D x D]}."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    G = Hv // Hk
    N = len(cu) - 1
    starts, ends = {}, {}
    Sf = np.zeros((N, Hv, dv, dk))
    dS0 = np.zeros((N, Hv, dv, dk))
    for n in range(N):
        chunks = _chunks(cu[n], cu[n + 1], C)
        segs = [chunks[i:i + seg] for i in range(0, len(chunks), seg)]
        for h in range(Hv):
            kh = h // G
            Q, K, V, gg, bb = scale * q[:, kh], k[:, kh], v[:, h], g[:, h], beta[:, h]
            Z = np.zeros((T, dk))
            B = [_run_chunks(sp, Q, K, V, gg, bb, np.zeros((dv, dk))) for sp in segs]
            Phi = [_run_chunks(sp, Q, K, Z, gg, bb, np.eye(dk)) for sp in segs]
            dB = [_rev_dS(sp, Q, K, V, gg, bb, dout[:, h], np.zeros((dv, dk))) for sp in segs]
            S = np.zeros((dv, dk)) if S0 is None else S0[n, h].astype(np.float64)
            starts[n, h] = []
            for s in range(len(segs)):
                starts[n, h].append(S)
                S = S @ Phi[s] + B[s]
            Sf[n, h] = S
            dS = np.zeros((dv, dk)) if dS_final is None else dS_final[n, h].astype(np.float64)
            ends[n, h] = [None] * len(segs)
            for s in reversed(range(len(segs))):
                ends[n, h][s] = dS
                dS = dS @ Phi[s].T + dB[s]
            dS0[n, h] = dS
    return starts, Sf, ends, dS0
