"""CPU oracle for the Gated DeltaNet layer core -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
may import this package.  The GPU library never links or calls it.

Thin ctypes wrapper over ``gdn_oracle.c`` (plain C, float64, token by token).
Every function here takes and returns float64 numpy arrays; it does no
arithmetic of its own except composing the per-op calls into a layer and the
optional round-to-bfloat16 at the layer's interface hand-offs (the rounding
helper comes from the shared input module).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

ACT_SILU = 0
ACT_SIGMOID = 1
L2_EPS = 1e-6
NORM_EPS = 1e-6
CONV_K = 4


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    D = ctypes.POINTER(ctypes.c_double)
    I = ctypes.POINTER(ctypes.c_int32)
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_conv_fwd.argtypes = [i64, i32, i32, D, D, I, i32, i32, i32, f64, D]
    lib.oracle_conv_bwd.argtypes = [i64, i32, i32, D, D, I, i32, i32, i32, f64, D, D, D]
    lib.oracle_conv_state_fwd.argtypes = [i64, i32, i32, D, D, I, i32, i32, i32, f64, D, D, D]
    lib.oracle_conv_state_bwd.argtypes = [i64, i32, i32, D, D, I, i32, i32, i32, f64, D, D, D, D,
                                          D, D]
    lib.oracle_gate_fwd.argtypes = [i64, i32, D, D, D, D, D, D]
    lib.oracle_gate_bwd.argtypes = [i64, i32, D, D, D, D, D, D, D, D, D, D]
    lib.oracle_delta_fwd.argtypes = [i64, i32, I, i32, i32, i32, i32, D, D, D, D, D, f64, D, D, D]
    lib.oracle_delta_bwd.argtypes = [i64, i32, I, i32, i32, i32, i32, D, D, D, D, D, f64, D, D, D,
                                     D, D, D, D, D, D]
    lib.oracle_norm_fwd.argtypes = [i64, i32, D, D, D, f64, ctypes.c_int, D]
    lib.oracle_norm_bwd.argtypes = [i64, i32, D, D, D, f64, ctypes.c_int, D, D, D, D]
    lib.oracle_max_threads.argtypes = []
    for name in ("oracle_conv_fwd", "oracle_conv_bwd", "oracle_conv_state_fwd",
                 "oracle_conv_state_bwd", "oracle_gate_fwd", "oracle_gate_bwd",
                 "oracle_delta_fwd", "oracle_delta_bwd", "oracle_norm_fwd", "oracle_norm_bwd",
                 "oracle_max_threads"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def threads() -> int:
    return int(_load().oracle_max_threads())


def _d(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _cu(cu):
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    return cu, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments")


# ---------------------------------------------------------------- conv
def conv_fwd(x, w, cu, n_l2: int, dk: int, eps: float = L2_EPS):
    """Causal depthwise conv (K taps) + SiLU + L2 over groups of dk among the
    first n_l2 channels.  x [T, C], w [C, K] -> y [T, C]."""
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    cu, cup = _cu(cu)
    y = np.empty_like(x)
    _check(_load().oracle_conv_fwd(T, C, w.shape[1], _d(x), _d(w), cup, len(cu) - 1, n_l2, dk,
                                   eps, _d(y)), "conv_fwd")
    return y


def conv_bwd(x, w, cu, n_l2: int, dk: int, dy, eps: float = L2_EPS):
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    T, C = x.shape
    cu, cup = _cu(cu)
    dx = np.empty_like(x)
    dw = np.empty_like(w)
    _check(_load().oracle_conv_bwd(T, C, w.shape[1], _d(x), _d(w), cup, len(cu) - 1, n_l2, dk,
                                   eps, _d(dy), _d(dx), _d(dw)), "conv_bwd")
    return dx, dw


def conv_state_fwd(x, w, cu, n_l2: int, dk: int, cs_in=None, eps: float = L2_EPS):
    """The convolution with a carried conv state: cs_in [N, K-1, C] holds the
    K-1 input rows before each sequence (None: zeros).  Returns y [T, C] and
    the final state [N, K-1, C] (the last K-1 input rows of each sequence,
    reaching into cs_in for short ones)."""
    x, w, cs_in = _f64(x), _f64(w), _f64(cs_in)
    T, C = x.shape
    K = w.shape[1]
    cu, cup = _cu(cu)
    N = len(cu) - 1
    y = np.empty_like(x)
    cs_out = np.empty((N, K - 1, C))
    _check(_load().oracle_conv_state_fwd(T, C, K, _d(x), _d(w), cup, N, n_l2, dk, eps, _d(cs_in),
                                         _d(y), _d(cs_out)), "conv_state_fwd")
    return y, cs_out


def conv_state_bwd(x, w, cu, n_l2: int, dk: int, dy, cs_in=None, dcs_out=None,
                   eps: float = L2_EPS):
    """Backward of conv_state_fwd: returns dx, dw, dcs_in."""
    x, w, dy, cs_in, dcs_out = _f64(x), _f64(w), _f64(dy), _f64(cs_in), _f64(dcs_out)
    T, C = x.shape
    K = w.shape[1]
    cu, cup = _cu(cu)
    N = len(cu) - 1
    dx = np.empty_like(x)
    dw = np.empty_like(w)
    dcs_in = np.empty((N, K - 1, C))
    _check(_load().oracle_conv_state_bwd(T, C, K, _d(x), _d(w), cup, N, n_l2, dk, eps, _d(cs_in),
                                         _d(dy), _d(dcs_out), _d(dx), _d(dw), _d(dcs_in)),
           "conv_state_bwd")
    return dx, dw, dcs_in


# ---------------------------------------------------------------- gate
def gate_fwd(a, b, A_log, dt_bias):
    a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
    T, H = a.shape
    g = np.empty_like(a)
    beta = np.empty_like(a)
    _check(_load().oracle_gate_fwd(T, H, _d(a), _d(b), _d(A_log), _d(dt_bias), _d(g), _d(beta)),
           "gate_fwd")
    return g, beta


def gate_bwd(a, b, A_log, dt_bias, dg, dbeta):
    a, b, A_log, dt_bias, dg, dbeta = map(_f64, (a, b, A_log, dt_bias, dg, dbeta))
    T, H = a.shape
    da, db = np.empty_like(a), np.empty_like(a)
    dA, ddt = np.empty(H), np.empty(H)
    _check(_load().oracle_gate_bwd(T, H, _d(a), _d(b), _d(A_log), _d(dt_bias), _d(dg), _d(dbeta),
                                   _d(da), _d(db), _d(dA), _d(ddt)), "gate_bwd")
    return da, db, dA, ddt


# ---------------------------------------------------------------- delta rule
def delta_fwd(q, k, v, g, beta, cu, scale: float, S0=None, want_final: bool = True):
    """q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv]; S0 [N, Hv, dv, dk].
    Returns o [T, Hv, dv] and S_final [N, Hv, dv, dk] (or None)."""
    q, k, v, g, beta, S0 = map(_f64, (q, k, v, g, beta, S0))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu, cup = _cu(cu)
    N = len(cu) - 1
    o = np.empty((T, Hv, dv))
    Sf = np.empty((N, Hv, dv, dk)) if want_final else None
    _check(_load().oracle_delta_fwd(T, N, cup, Hk, Hv, dk, dv, _d(q), _d(k), _d(v), _d(g),
                                    _d(beta), scale, _d(S0), _d(o), _d(Sf)), "delta_fwd")
    return o, Sf


def delta_bwd(q, k, v, g, beta, cu, scale: float, dout, S0=None, dS_final=None):
    """Returns dq, dk [T, Hk, dk], dv [T, Hv, dv], dg, dbeta [T, Hv], dS0 [N, Hv, dv, dk]."""
    q, k, v, g, beta, S0, dout, dS_final = map(_f64, (q, k, v, g, beta, S0, dout, dS_final))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    cu, cup = _cu(cu)
    N = len(cu) - 1
    dq, dkk = np.empty_like(q), np.empty_like(k)
    dvv = np.empty_like(v)
    dg, dbeta = np.empty((T, Hv)), np.empty((T, Hv))
    dS0 = np.empty((N, Hv, dv, dk))
    _check(_load().oracle_delta_bwd(T, N, cup, Hk, Hv, dk, dv, _d(q), _d(k), _d(v), _d(g),
                                    _d(beta), scale, _d(S0), _d(dout), _d(dS_final), _d(dq),
                                    _d(dkk), _d(dvv), _d(dg), _d(dbeta), _d(dS0)), "delta_bwd")
    return dq, dkk, dvv, dg, dbeta, dS0


# ---------------------------------------------------------------- gated norm
def norm_fwd(o, z, w, act: int = ACT_SILU, eps: float = NORM_EPS):
    """Rows over the last axis of o, z.  w [d]."""
    o, z, w = _f64(o), _f64(z), _f64(w)
    d = o.shape[-1]
    rows = o.size // d
    y = np.empty_like(o)
    _check(_load().oracle_norm_fwd(rows, d, _d(o), _d(z), _d(w), eps, act, _d(y)), "norm_fwd")
    return y


def norm_bwd(o, z, w, dy, act: int = ACT_SILU, eps: float = NORM_EPS):
    o, z, w, dy = _f64(o), _f64(z), _f64(w), _f64(dy)
    d = o.shape[-1]
    rows = o.size // d
    do, dz = np.empty_like(o), np.empty_like(o)
    dw = np.empty(d)
    _check(_load().oracle_norm_bwd(rows, d, _d(o), _d(z), _d(w), eps, act, _d(dy), _d(do), _d(dz),
                                   _d(dw)), "norm_bwd")
    return do, dz, dw


# ---------------------------------------------------------------- layer
def _split(y, hk, hv, d):
    T = y.shape[0]
    return (y[:, : hk * d].reshape(T, hk, d), y[:, hk * d: 2 * hk * d].reshape(T, hk, d),
            y[:, 2 * hk * d:].reshape(T, hv, d))


def layer_fwd(inp: dict, hk: int, hv: int, d: int, scale: float, act: int = ACT_SILU,
              round_fn=None):
    """conv -> gate -> gated delta rule -> gated norm, each an oracle call.

    ``round_fn`` (optional) is applied to the conv output and to the delta
    rule output, the two token tensors the layer hands between its calls in
    the storage dtype.  Returns a dict of every intermediate."""
    rf = (lambda a: a) if round_fn is None else round_fn
    cu = inp["cu_seqlens"]
    cs_out = None
    if inp.get("conv_state") is not None:    # carried conv state in and out
        y, cs_out = conv_state_fwd(inp["x"], inp["w_conv"], cu, 2 * hk * d, d, inp["conv_state"])
        y = rf(y)
    else:
        y = rf(conv_fwd(inp["x"], inp["w_conv"], cu, 2 * hk * d, d))
    q, k, v = _split(y, hk, hv, d)
    g, beta = gate_fwd(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    o, Sf = delta_fwd(q, k, v, g, beta, cu, scale, inp.get("S0"))
    o = rf(o)
    out = norm_fwd(o, inp["z"], inp["w_norm"], act)
    return {"y": y, "q": q, "k": k, "v": v, "g": g, "beta": beta, "o": o, "S_final": Sf,
            "out": out, "conv_state_out": cs_out}


def layer_bwd(inp: dict, fwd: dict, hk: int, hv: int, d: int, scale: float, act: int = ACT_SILU,
              round_fn=None):
    """Backward of layer_fwd given the upstream gradient inp['dy'] (and
    inp['dS_T'] for the final state).  Gradients handed between calls in the
    storage dtype pass through ``round_fn``."""
    rf = (lambda a: a) if round_fn is None else round_fn
    cu = inp["cu_seqlens"]
    T = inp["x"].shape[0]
    do, dz, dw_norm = norm_bwd(fwd["o"], inp["z"], inp["w_norm"], inp["dy"], act)
    do = rf(do)
    dq, dk, dv, dg, dbeta, dS0 = delta_bwd(fwd["q"], fwd["k"], fwd["v"], fwd["g"], fwd["beta"], cu,
                                           scale, do, inp.get("S0"), inp.get("dS_T"))
    dy_conv = rf(np.concatenate([dq.reshape(T, -1), dk.reshape(T, -1), dv.reshape(T, -1)], axis=1))
    da, db, dA_log, ddt_bias = gate_bwd(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], dg, dbeta)
    dcs_in = None
    if inp.get("conv_state") is not None:    # carried conv state (and its gradient d_conv_state)
        dx, dw_conv, dcs_in = conv_state_bwd(inp["x"], inp["w_conv"], cu, 2 * hk * d, d, dy_conv,
                                             inp["conv_state"], inp.get("d_conv_state"))
    else:
        dx, dw_conv = conv_bwd(inp["x"], inp["w_conv"], cu, 2 * hk * d, d, dy_conv)
    return {"do": do, "dz": dz, "dw_norm": dw_norm, "dq": dq, "dk": dk, "dv": dv, "dg": dg,
            "dbeta": dbeta, "dS0": dS0, "dy_conv": dy_conv, "da": da, "db": db,
            "dA_log": dA_log, "ddt_bias": ddt_bias, "dx": dx, "dw_conv": dw_conv,
            "d_conv_state": dcs_in}


# ---------------------------------------------------------------------------
# The layer with its projections: hidden states X [T, H] go through plain
# products to the core's inputs (x = X W_x^T with the q | k | v channels,
# z = X W_z^T, a = X W_a^T, b = X W_b^T), the core runs as layer_fwd, and its
# gated-norm output leaves through Y = out W_out^T.  The projections are the
# plain definition (numpy products in fp64); ``round_fn`` marks the tensors
# handed between calls in the storage dtype, as in layer_fwd.
def proj_layer_fwd(X, W: dict, params: dict, cu, hk: int, hv: int, d: int, scale: float,
                   act: int = ACT_SILU, round_fn=None, S0=None):
    rf = (lambda a: a) if round_fn is None else round_fn
    X = _f64(X)
    T = X.shape[0]
    inp = {"x": rf(X @ _f64(W["x"]).T), "z": rf(X @ _f64(W["z"]).T).reshape(T, hv, d),
           "a": rf(X @ _f64(W["a"]).T), "b": rf(X @ _f64(W["b"]).T), "cu_seqlens": cu, "S0": S0}
    inp.update(params)
    f = layer_fwd(inp, hk, hv, d, scale, act, round_fn)
    out = rf(f["out"]).reshape(T, hv * d)
    f.update(inp=inp, out_flat=out, Y=out @ _f64(W["out"]).T)
    return f


def proj_layer_bwd(X, W: dict, fwd: dict, dY, hk: int, hv: int, d: int, scale: float,
                   act: int = ACT_SILU, round_fn=None, dS_T=None):
    """Backward of proj_layer_fwd for the upstream gradient dY [T, H]: the
    core's backward between the products' transposes.  Weight gradients are
    dW = (gradient of the product's output)^T (its input)."""
    rf = (lambda a: a) if round_fn is None else round_fn
    X, dY = _f64(X), _f64(dY)
    T = X.shape[0]
    inp = dict(fwd["inp"])
    inp["dy"] = rf(dY @ _f64(W["out"])).reshape(T, hv, d)
    inp["dS_T"] = dS_T
    g = layer_bwd(inp, fwd, hk, hv, d, scale, act, round_fn)
    gx, gz = g["dx"], g["dz"].reshape(T, hv * d)
    ga, gb = g["da"], g["db"]
    g["dX"] = gx @ _f64(W["x"]) + gz @ _f64(W["z"]) + ga @ _f64(W["a"]) + gb @ _f64(W["b"])
    g["dW"] = {"x": gx.T @ X, "z": gz.T @ X, "a": ga.T @ X, "b": gb.T @ X,
               "out": dY.T @ fwd["out_flat"]}
    return g

