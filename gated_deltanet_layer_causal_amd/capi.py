"""ctypes binding of libgdn.so: the C ABI in include/libgdn.h, one Python
function per exported entry point, same names.

Argument marshalling only: tensors are torch CUDA (HIP) tensors, passed as
raw device pointers with their row strides; the stream is torch's current
stream unless one is given.  All arithmetic happens in the HIP kernels.
There is no fallback: if the library is missing, was built from other
sources than those in the tree, or a call fails, an error is raised.

The C side takes most tensors without strides and cannot see their sizes, so
every wrapper checks dtype, device, layout and element count against the
shape before the call: a caller's mistake becomes a Python exception rather
than an out-of-bounds device access.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_BF16, GDN_FP32, GDN_FP16 = 0, 1, 2
GDN_ACT_SILU, GDN_ACT_SIGMOID = 0, 1
EXPORTS = (
    "gdn_status_string", "gdn_conv_fwd", "gdn_conv_bwd", "gdn_conv_bwd_workspace",
    "gdn_conv_bwd_noalloc", "gdn_conv_fwd_state", "gdn_conv_bwd_state", "gdn_gate_fwd",
    "gdn_gate_bwd", "gdn_gate_bwd_workspace", "gdn_chunk_fwd", "gdn_chunk_fwd_workspace",
    "gdn_chunk_bwd", "gdn_chunk_bwd_workspace", "gdn_gated_norm_fwd", "gdn_gated_norm_bwd",
    "gdn_gated_norm_bwd_workspace", "gdn_chunk_prepare", "gdn_chunk_prepare_bwd",
    "gdn_chunk_fwd_states", "gdn_chunk_fwd_states_save",
    "gdn_chunk_bwd_states", "gdn_chunk_bwd_reverse", "gdn_chunk_bwd_grads",
    "gdn_check_cu_seqlens",
)


class Shape(ctypes.Structure):
    _fields_ = [("n_seq", c_int32), ("total_tokens", c_int64), ("hk", c_int32), ("hv", c_int32),
                ("dk", c_int32), ("dv", c_int32), ("conv_k", c_int32), ("chunk", c_int32),
                ("dtype", c_int), ("seg_chunks", c_int32)]


class GDNError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed: status {status} ({msg})")
        self.status = status


_lib = None


def _check_built(path: str):
    from . import build as _b
    hint = "build it first: python -c 'import __graft_entry__ as g; g.build()'"
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; {hint}")
    dig = path + ".sources"
    have = open(dig).read().strip() if os.path.exists(dig) else None
    if have != _b.source_digest():
        raise RuntimeError(f"{path} was not built from the HIP sources in this tree; {hint}")


def load(path: str = LIB_PATH):
    """Load libgdn.so; refuses a missing library or one built from other
    sources (the digest written by build.py must match csrc/ and include/)."""
    global _lib
    if _lib is not None:
        return _lib
    _check_built(path)
    lib = ctypes.CDLL(path)
    SP = POINTER(Shape)
    V, I64, F = c_void_p, c_int64, c_float
    lib.gdn_status_string.argtypes = [c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_conv_fwd.argtypes = [SP, V, I64, V, V, c_int, F, V, I64, V]
    lib.gdn_conv_bwd.argtypes = [SP, V, I64, V, V, c_int, F, V, I64, V, I64, V, V, c_size_t, V]
    lib.gdn_conv_bwd_noalloc.argtypes = [SP, V, I64, V, V, c_int, F, V, I64, V, I64, V, V]
    lib.gdn_conv_fwd_state.argtypes = [SP, V, I64, V, V, c_int, F, V, V, I64, V, V]
    lib.gdn_conv_bwd_state.argtypes = [SP, V, I64, V, V, c_int, F, V, V, I64, V, V, I64, V, V, V,
                                       c_size_t, V]
    lib.gdn_gate_fwd.argtypes = [SP, V, V, V, V, V, V, V]
    lib.gdn_gate_bwd.argtypes = [SP, V, V, V, V, V, V, V, V, V, V, V, c_size_t, V]
    lib.gdn_chunk_fwd.argtypes = [SP, V, V, V, I64, I64, I64, V, V, F, V, V, V, V, V, c_size_t, V]
    lib.gdn_chunk_bwd.argtypes = [SP, V, V, V, I64, I64, I64, V, V, F, V, V, V, V, V, V, V, I64,
                                  I64, I64, V, V, V, V, c_size_t, V]
    lib.gdn_chunk_prepare.argtypes = [SP, V, V, I64, I64, V, V, F, V, V, c_size_t, V]
    lib.gdn_chunk_prepare_bwd.argtypes = [SP, V, V, I64, I64, V, V, F, V, V, c_size_t, V]
    lib.gdn_chunk_fwd_states.argtypes = [SP, V, V, V, I64, I64, I64, F, V, V, V, V, V, c_size_t, V]
    lib.gdn_chunk_fwd_states_save.argtypes = lib.gdn_chunk_fwd_states.argtypes
    lib.gdn_chunk_bwd_states.argtypes = [SP, V, V, V, I64, I64, I64, F, V, V, V, c_size_t, V]
    lib.gdn_chunk_bwd_reverse.argtypes = [SP, V, V, I64, I64, F, V, V, V, V, I64, V, V, c_size_t, V]
    lib.gdn_chunk_bwd_grads.argtypes = [SP, V, V, I64, I64, V, F, V, V, V, I64, V, V, I64, I64, V,
                                        V, V, c_size_t, V]
    lib.gdn_gated_norm_fwd.argtypes = [I64, c_int32, c_int, V, V, V, F, c_int, V, V]
    lib.gdn_check_cu_seqlens.argtypes = [SP, V, V, V]
    lib.gdn_gated_norm_bwd.argtypes = [I64, c_int32, c_int, V, V, V, F, c_int, V, V, V, V, V,
                                       c_size_t, V]
    for name in ("gdn_conv_bwd_workspace", "gdn_gate_bwd_workspace", "gdn_chunk_fwd_workspace",
                 "gdn_chunk_bwd_workspace"):
        getattr(lib, name).argtypes = [SP]
        getattr(lib, name).restype = c_size_t
    lib.gdn_gated_norm_bwd_workspace.argtypes = [I64, c_int32]
    lib.gdn_gated_norm_bwd_workspace.restype = c_size_t
    for name in ("gdn_conv_fwd", "gdn_conv_bwd", "gdn_conv_bwd_noalloc", "gdn_conv_fwd_state",
                 "gdn_conv_bwd_state", "gdn_gate_fwd", "gdn_gate_bwd", "gdn_chunk_fwd",
                 "gdn_chunk_bwd", "gdn_gated_norm_fwd", "gdn_gated_norm_bwd", "gdn_chunk_prepare",
                 "gdn_chunk_prepare_bwd", "gdn_chunk_fwd_states", "gdn_chunk_fwd_states_save",
                 "gdn_chunk_bwd_states", "gdn_chunk_bwd_reverse",
                 "gdn_chunk_bwd_grads", "gdn_check_cu_seqlens"):
        getattr(lib, name).restype = c_int
    _lib = lib
    return lib


def _p(t):
    """The device pointer of a tensor (None for None); host tensors are
    refused here, after the wrappers' dtype and size checks."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libgdn takes device tensors only; got a host tensor")
    return c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _ok(name, st):
    if st != 0:
        raise GDNError(name, st, load().gdn_status_string(st).decode())


_GDN_DT = {torch.bfloat16: GDN_BF16, torch.float32: GDN_FP32, torch.float16: GDN_FP16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _GDN_DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _GDN_DT[t.dtype]


def make_shape(n_seq, total_tokens, hk, hv, d, dtype, seg_chunks=0) -> Shape:
    """seg_chunks: segment length of the segment-parallel state scan (0: the
    library decides, > 0: forced, < 0: one sequential pass per sequence)."""
    dt = dtype if isinstance(dtype, int) else _GDN_DT[dtype]
    return Shape(n_seq, total_tokens, hk, hv, d, d, 4, 64, dt, seg_chunks)


def _ld(t):
    return t.stride(0) if t.dim() > 0 else 0


# ---------------------------------------------------------------- workspace queries
def gdn_conv_bwd_workspace(shape):
    return int(load().gdn_conv_bwd_workspace(byref(shape)))


def gdn_gate_bwd_workspace(shape):
    return int(load().gdn_gate_bwd_workspace(byref(shape)))


def gdn_chunk_fwd_workspace(shape):
    return int(load().gdn_chunk_fwd_workspace(byref(shape)))


def gdn_chunk_bwd_workspace(shape):
    return int(load().gdn_chunk_bwd_workspace(byref(shape)))


def gdn_gated_norm_bwd_workspace(rows, dv):
    return int(load().gdn_gated_norm_bwd_workspace(rows, dv))


# ---------------------------------------------------------------- argument checks
_TDT = {GDN_BF16: torch.bfloat16, GDN_FP32: torch.float32, GDN_FP16: torch.float16}


def _tdt(shape) -> torch.dtype:
    return _TDT[shape.dtype]


def _need(name, t, dtype, numel=None, optional=False):
    """A contiguous device tensor of `dtype` with `numel` elements (or None
    when optional)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the shape needs {numel}")


def _rows(name, t, dtype, T, cols):
    """A [T, cols] device matrix of `dtype` with contiguous rows (any row
    stride; the C side checks its alignment)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (T, cols) or (T > 0 and cols > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a [{T}, {cols}] matrix with contiguous rows, got "
                         f"shape {tuple(t.shape)} strides {t.stride()}")


def _ws(ws):
    if ws is None:
        return
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")


def _cu_ok(shape, cu):
    _need("cu_seqlens", cu, torch.int32, shape.n_seq + 1)


def _state(name, shape, t, optional=True):
    _need(name, t, torch.float32, shape.n_seq * shape.hv * shape.dk * shape.dv, optional=optional)


def _chunk_qk(shape, q, k):
    _rows("q", q, _tdt(shape), shape.total_tokens, shape.hk * shape.dk)
    _rows("k", k, _tdt(shape), shape.total_tokens, shape.hk * shape.dk)


def _per_token(name, shape, t, dtype=torch.float32):
    _need(name, t, dtype, shape.total_tokens * shape.hv)


def _heads(name, shape, t):
    _need(name, t, _tdt(shape), shape.total_tokens * shape.hv * shape.dv)


def _conv_ok(shape, x, w, cu):
    C = 2 * shape.hk * shape.dk + shape.hv * shape.dv
    _rows("x", x, _tdt(shape), shape.total_tokens, C)
    _need("w", w, torch.float32, C * 4)
    _cu_ok(shape, cu)
    return C


# ---------------------------------------------------------------- entry points
def gdn_conv_fwd(shape, x, w, cu_seqlens, y, l2norm_qk=True, l2_eps=1e-6, stream=None):
    C = _conv_ok(shape, x, w, cu_seqlens)
    _rows("y", y, _tdt(shape), shape.total_tokens, C)
    _ok("gdn_conv_fwd", load().gdn_conv_fwd(byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens),
                                            int(l2norm_qk), l2_eps, _p(y), _ld(y), _stream(stream)))


def gdn_conv_bwd(shape, x, w, cu_seqlens, dy, dx, dw, ws, l2norm_qk=True, l2_eps=1e-6,
                 stream=None):
    C = _conv_ok(shape, x, w, cu_seqlens)
    _rows("dy", dy, _tdt(shape), shape.total_tokens, C)
    _rows("dx", dx, _tdt(shape), shape.total_tokens, C)
    _need("dw", dw, torch.float32, C * 4)
    _ws(ws)
    _ok("gdn_conv_bwd", load().gdn_conv_bwd(byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens),
                                            int(l2norm_qk), l2_eps, _p(dy), _ld(dy), _p(dx),
                                            _ld(dx), _p(dw), _p(ws), ws.numel() if ws is not None else 0,
                                            _stream(stream)))


def _conv_state(name, shape, t):
    _need(name, t, _tdt(shape), shape.n_seq * 3 * (2 * shape.hk * shape.dk + shape.hv * shape.dv),
          optional=True)


def gdn_conv_fwd_state(shape, x, w, cu_seqlens, y, conv_state_in=None, conv_state_out=None,
                       l2norm_qk=True, l2_eps=1e-6, stream=None):
    C = _conv_ok(shape, x, w, cu_seqlens)
    _rows("y", y, _tdt(shape), shape.total_tokens, C)
    _conv_state("conv_state_in", shape, conv_state_in)
    _conv_state("conv_state_out", shape, conv_state_out)
    _ok("gdn_conv_fwd_state", load().gdn_conv_fwd_state(
        byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens), int(l2norm_qk), l2_eps,
        _p(conv_state_in), _p(y), _ld(y), _p(conv_state_out), _stream(stream)))


def gdn_conv_bwd_state(shape, x, w, cu_seqlens, dy, dx, dw, ws, conv_state_in=None,
                       d_conv_state_out=None, d_conv_state_in=None, l2norm_qk=True, l2_eps=1e-6,
                       stream=None):
    C = _conv_ok(shape, x, w, cu_seqlens)
    _rows("dy", dy, _tdt(shape), shape.total_tokens, C)
    _rows("dx", dx, _tdt(shape), shape.total_tokens, C)
    _need("dw", dw, torch.float32, C * 4)
    for nm, t in (("conv_state_in", conv_state_in), ("d_conv_state_out", d_conv_state_out),
                  ("d_conv_state_in", d_conv_state_in)):
        _conv_state(nm, shape, t)
    _ws(ws)
    _ok("gdn_conv_bwd_state", load().gdn_conv_bwd_state(
        byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens), int(l2norm_qk), l2_eps,
        _p(conv_state_in), _p(dy), _ld(dy), _p(d_conv_state_out), _p(dx), _ld(dx), _p(dw),
        _p(d_conv_state_in), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)))


CONV_BWD_NOALLOC_MAX_BYTES = 32 << 20   # GDN_CONV_BWD_NOALLOC_MAX_BYTES in libgdn.h


def gdn_conv_bwd_noalloc(shape, x, w, cu_seqlens, dy, dx, dw, l2norm_qk=True, l2_eps=1e-6,
                         stream=None):
    """gdn_conv_bwd with the library's own scratch (no workspace, no
    allocation); see libgdn.h for its size limit and sharing rules."""
    C = _conv_ok(shape, x, w, cu_seqlens)
    _rows("dy", dy, _tdt(shape), shape.total_tokens, C)
    _rows("dx", dx, _tdt(shape), shape.total_tokens, C)
    _need("dw", dw, torch.float32, C * 4)
    _ok("gdn_conv_bwd_noalloc", load().gdn_conv_bwd_noalloc(
        byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens), int(l2norm_qk), l2_eps, _p(dy),
        _ld(dy), _p(dx), _ld(dx), _p(dw), _stream(stream)))


def _gate_ok(shape, a, b, A_log, dt_bias):
    _per_token("a", shape, a, _tdt(shape))
    _per_token("b", shape, b, _tdt(shape))
    _need("A_log", A_log, torch.float32, shape.hv)
    _need("dt_bias", dt_bias, torch.float32, shape.hv)


CU_BAD_START, CU_BAD_END, CU_DECREASING = 1, 2, 4


def gdn_check_cu_seqlens(shape, cu_seqlens, violations, stream=None):
    """Writes to violations (an int32 device tensor of one element) the bit
    mask of the cu_seqlens contract's violations (CU_BAD_START, CU_BAD_END,
    CU_DECREASING; 0 when valid), asynchronously."""
    _cu_ok(shape, cu_seqlens)
    _need("violations", violations, torch.int32, 1)
    _ok("gdn_check_cu_seqlens", load().gdn_check_cu_seqlens(byref(shape), _p(cu_seqlens),
                                                            _p(violations), _stream(stream)))


def gdn_gate_fwd(shape, a, b, A_log, dt_bias, g, beta, stream=None):
    _gate_ok(shape, a, b, A_log, dt_bias)
    _per_token("g", shape, g)
    _per_token("beta", shape, beta)
    _ok("gdn_gate_fwd", load().gdn_gate_fwd(byref(shape), _p(a), _p(b), _p(A_log), _p(dt_bias),
                                            _p(g), _p(beta), _stream(stream)))


def gdn_gate_bwd(shape, a, b, A_log, dt_bias, dg, dbeta, da, db, dA_log, ddt_bias, ws,
                 stream=None):
    _gate_ok(shape, a, b, A_log, dt_bias)
    for nm, t in (("dg", dg), ("dbeta", dbeta)):
        _per_token(nm, shape, t)
    for nm, t in (("da", da), ("db", db)):
        _per_token(nm, shape, t, _tdt(shape))
    _need("dA_log", dA_log, torch.float32, shape.hv)
    _need("ddt_bias", ddt_bias, torch.float32, shape.hv)
    _ws(ws)
    _ok("gdn_gate_bwd", load().gdn_gate_bwd(byref(shape), _p(a), _p(b), _p(A_log), _p(dt_bias),
                                            _p(dg), _p(dbeta), _p(da), _p(db), _p(dA_log),
                                            _p(ddt_bias), _p(ws), ws.numel() if ws is not None else 0,
                                            _stream(stream)))


def _chunk_fwd_ok(shape, q, k, v, g, beta, S0, S_final, cu, o, ws):
    _chunk_qk(shape, q, k)
    _rows("v", v, _tdt(shape), shape.total_tokens, shape.hv * shape.dv)
    if g is not None or beta is not None:
        _per_token("g", shape, g)
        _per_token("beta", shape, beta)
    _state("S0", shape, S0)
    _state("S_final", shape, S_final)
    _cu_ok(shape, cu)
    if o is not None:
        _heads("o", shape, o)
    _ws(ws)


def gdn_chunk_fwd(shape, q, k, v, g, beta, scale, S0, S_final, cu_seqlens, o, ws, stream=None):
    _chunk_fwd_ok(shape, q, k, v, g, beta, S0, S_final, cu_seqlens, o, ws)
    _per_token("g", shape, g)
    _per_token("beta", shape, beta)
    _heads("o", shape, o)
    _ok("gdn_chunk_fwd", load().gdn_chunk_fwd(byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k),
                                              _ld(v), _p(g), _p(beta), scale, _p(S0), _p(S_final),
                                              _p(cu_seqlens), _p(o), _p(ws), ws.numel(),
                                              _stream(stream)))


def _chunk_grads_ok(shape, dq, dk, dg, dbeta):
    _rows("dq", dq, _tdt(shape), shape.total_tokens, shape.hk * shape.dk)
    _rows("dk", dk, _tdt(shape), shape.total_tokens, shape.hk * shape.dk)
    _per_token("dg", shape, dg)
    _per_token("dbeta", shape, dbeta)


def gdn_chunk_bwd(shape, q, k, v, g, beta, scale, S0, cu_seqlens, dout, dS_final, dq, dk, dv, dg,
                  dbeta, dS0, ws, stream=None):
    _chunk_fwd_ok(shape, q, k, v, g, beta, S0, None, cu_seqlens, None, ws)
    _per_token("g", shape, g)
    _per_token("beta", shape, beta)
    _heads("dout", shape, dout)
    _state("dS_final", shape, dS_final)
    _state("dS0", shape, dS0)
    _chunk_grads_ok(shape, dq, dk, dg, dbeta)
    _rows("dv", dv, _tdt(shape), shape.total_tokens, shape.hv * shape.dv)
    _ok("gdn_chunk_bwd", load().gdn_chunk_bwd(byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k),
                                              _ld(v), _p(g), _p(beta), scale, _p(S0),
                                              _p(cu_seqlens), _p(dout), _p(dS_final), _p(dq),
                                              _p(dk), _p(dv), _ld(dq), _ld(dk), _ld(dv), _p(dg),
                                              _p(dbeta), _p(dS0), _p(ws), ws.numel(),
                                              _stream(stream)))


def _prep_ok(shape, q, k, g, beta, cu, ws):
    _chunk_qk(shape, q, k)
    _per_token("g", shape, g)
    _per_token("beta", shape, beta)
    _cu_ok(shape, cu)
    _ws(ws)


def gdn_chunk_prepare(shape, q, k, g, beta, scale, cu_seqlens, ws, stream=None):
    _prep_ok(shape, q, k, g, beta, cu_seqlens, ws)
    _ok("gdn_chunk_prepare", load().gdn_chunk_prepare(byref(shape), _p(q), _p(k), _ld(q), _ld(k),
                                                      _p(g), _p(beta), scale, _p(cu_seqlens),
                                                      _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_prepare_bwd(shape, q, k, g, beta, scale, cu_seqlens, ws, stream=None):
    _prep_ok(shape, q, k, g, beta, cu_seqlens, ws)
    _ok("gdn_chunk_prepare_bwd", load().gdn_chunk_prepare_bwd(
        byref(shape), _p(q), _p(k), _ld(q), _ld(k), _p(g), _p(beta), scale, _p(cu_seqlens), _p(ws),
        ws.numel(), _stream(stream)))


def gdn_chunk_fwd_states(shape, q, k, v, scale, S0, S_final, cu_seqlens, o, ws, stream=None):
    _chunk_fwd_ok(shape, q, k, v, None, None, S0, S_final, cu_seqlens, o, ws)
    _heads("o", shape, o)
    _ok("gdn_chunk_fwd_states", load().gdn_chunk_fwd_states(
        byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k), _ld(v), scale, _p(S0), _p(S_final),
        _p(cu_seqlens), _p(o), _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_fwd_states_save(shape, q, k, v, scale, S0, S_final, cu_seqlens, o, ws, stream=None):
    _chunk_fwd_ok(shape, q, k, v, None, None, S0, S_final, cu_seqlens, o, ws)
    _heads("o", shape, o)
    _ok("gdn_chunk_fwd_states_save", load().gdn_chunk_fwd_states_save(
        byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k), _ld(v), scale, _p(S0), _p(S_final),
        _p(cu_seqlens), _p(o), _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_bwd_states(shape, q, k, v, scale, S0, cu_seqlens, ws, stream=None):
    _chunk_fwd_ok(shape, q, k, v, None, None, S0, None, cu_seqlens, None, ws)
    _ok("gdn_chunk_bwd_states", load().gdn_chunk_bwd_states(
        byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k), _ld(v), scale, _p(S0), _p(cu_seqlens),
        _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_bwd_reverse(shape, q, k, scale, cu_seqlens, dout, dS_final, dv, dS0, ws, stream=None):
    _chunk_qk(shape, q, k)
    _cu_ok(shape, cu_seqlens)
    _heads("dout", shape, dout)
    _state("dS_final", shape, dS_final)
    _state("dS0", shape, dS0)
    _rows("dv", dv, _tdt(shape), shape.total_tokens, shape.hv * shape.dv)
    _ws(ws)
    _ok("gdn_chunk_bwd_reverse", load().gdn_chunk_bwd_reverse(
        byref(shape), _p(q), _p(k), _ld(q), _ld(k), scale, _p(cu_seqlens), _p(dout), _p(dS_final),
        _p(dv), _ld(dv), _p(dS0), _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_bwd_grads(shape, q, k, beta, scale, cu_seqlens, dout, dv, dq, dk, dg, dbeta, ws,
                        stream=None):
    _chunk_qk(shape, q, k)
    _per_token("beta", shape, beta)
    _cu_ok(shape, cu_seqlens)
    _heads("dout", shape, dout)
    _rows("dv", dv, _tdt(shape), shape.total_tokens, shape.hv * shape.dv)
    _chunk_grads_ok(shape, dq, dk, dg, dbeta)
    _ws(ws)
    _ok("gdn_chunk_bwd_grads", load().gdn_chunk_bwd_grads(
        byref(shape), _p(q), _p(k), _ld(q), _ld(k), _p(beta), scale, _p(cu_seqlens), _p(dout),
        _p(dv), _ld(dv), _p(dq), _p(dk), _ld(dq), _ld(dk), _p(dg), _p(dbeta), _p(ws), ws.numel(),
        _stream(stream)))


def _norm_ok(o, z, w, *others):
    dv = o.shape[-1]
    rows = o.numel() // dv if dv else 0
    dt = o.dtype
    _need("o", o, dt, rows * dv)
    _need("z", z, dt, rows * dv)
    for nm, t in others:
        _need(nm, t, dt, rows * dv)
    _need("w", w, torch.float32, dv)
    return rows, dv


def gdn_gated_norm_fwd(o, z, w, y, eps=1e-6, act=GDN_ACT_SILU, stream=None):
    rows, dv = _norm_ok(o, z, w, ("y", y))
    _ok("gdn_gated_norm_fwd", load().gdn_gated_norm_fwd(rows, dv, _dt(o), _p(o), _p(z), _p(w), eps,
                                                        act, _p(y), _stream(stream)))


def gdn_gated_norm_bwd(o, z, w, dy, dout, dz, dw, ws, eps=1e-6, act=GDN_ACT_SILU, stream=None):
    rows, dv = _norm_ok(o, z, w, ("dy", dy), ("dout", dout), ("dz", dz))
    _need("dw", dw, torch.float32, dv)
    _ws(ws)
    _ok("gdn_gated_norm_bwd", load().gdn_gated_norm_bwd(rows, dv, _dt(o), _p(o), _p(z), _p(w), eps,
                                                        act, _p(dy), _p(dout), _p(dz), _p(dw),
                                                        _p(ws), ws.numel(), _stream(stream)))
