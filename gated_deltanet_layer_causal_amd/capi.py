"""ctypes binding of libgdn.so: the C ABI in include/libgdn.h, one Python
function per exported entry point, same names.

Argument marshalling only: tensors are torch CUDA (HIP) tensors, passed as
raw device pointers with their row strides; the stream is torch's current
stream unless one is given.  All arithmetic happens in the HIP kernels.
There is no fallback: if the library is missing or a call fails, an error is
raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_BF16, GDN_FP32 = 0, 1
GDN_ACT_SILU, GDN_ACT_SIGMOID = 0, 1
EXPORTS = (
    "gdn_status_string", "gdn_conv_fwd", "gdn_conv_bwd", "gdn_conv_bwd_workspace", "gdn_gate_fwd",
    "gdn_gate_bwd", "gdn_gate_bwd_workspace", "gdn_chunk_fwd", "gdn_chunk_fwd_workspace",
    "gdn_chunk_bwd", "gdn_chunk_bwd_workspace", "gdn_gated_norm_fwd", "gdn_gated_norm_bwd",
    "gdn_gated_norm_bwd_workspace", "gdn_chunk_prepare", "gdn_chunk_prepare_bwd",
    "gdn_chunk_fwd_states", "gdn_chunk_fwd_states_save",
    "gdn_chunk_bwd_states", "gdn_chunk_bwd_reverse", "gdn_chunk_bwd_grads",
)


class Shape(ctypes.Structure):
    _fields_ = [("n_seq", c_int32), ("total_tokens", c_int64), ("hk", c_int32), ("hv", c_int32),
                ("dk", c_int32), ("dv", c_int32), ("conv_k", c_int32), ("chunk", c_int32),
                ("dtype", c_int)]


class GDNError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed: status {status} ({msg})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libgdn.so (building it first only if no library exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    SP = POINTER(Shape)
    V, I64, F = c_void_p, c_int64, c_float
    lib.gdn_status_string.argtypes = [c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_conv_fwd.argtypes = [SP, V, I64, V, V, c_int, F, V, I64, V]
    lib.gdn_conv_bwd.argtypes = [SP, V, I64, V, V, c_int, F, V, I64, V, I64, V, V, c_size_t, V]
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
    lib.gdn_gated_norm_bwd.argtypes = [I64, c_int32, c_int, V, V, V, F, c_int, V, V, V, V, V,
                                       c_size_t, V]
    for name in ("gdn_conv_bwd_workspace", "gdn_gate_bwd_workspace", "gdn_chunk_fwd_workspace",
                 "gdn_chunk_bwd_workspace"):
        getattr(lib, name).argtypes = [SP]
        getattr(lib, name).restype = c_size_t
    lib.gdn_gated_norm_bwd_workspace.argtypes = [I64, c_int32]
    lib.gdn_gated_norm_bwd_workspace.restype = c_size_t
    for name in ("gdn_conv_fwd", "gdn_conv_bwd", "gdn_gate_fwd", "gdn_gate_bwd", "gdn_chunk_fwd",
                 "gdn_chunk_bwd", "gdn_gated_norm_fwd", "gdn_gated_norm_bwd", "gdn_chunk_prepare",
                 "gdn_chunk_prepare_bwd", "gdn_chunk_fwd_states", "gdn_chunk_fwd_states_save",
                 "gdn_chunk_bwd_states", "gdn_chunk_bwd_reverse",
                 "gdn_chunk_bwd_grads"):
        getattr(lib, name).restype = c_int
    _lib = lib
    return lib


def _p(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _ok(name, st):
    if st != 0:
        raise GDNError(name, st, load().gdn_status_string(st).decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_shape(n_seq, total_tokens, hk, hv, d, dtype) -> Shape:
    dt = dtype if isinstance(dtype, int) else (GDN_BF16 if dtype == torch.bfloat16 else GDN_FP32)
    return Shape(n_seq, total_tokens, hk, hv, d, d, 4, 64, dt)


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


# ---------------------------------------------------------------- entry points
def gdn_conv_fwd(shape, x, w, cu_seqlens, y, l2norm_qk=True, l2_eps=1e-6, stream=None):
    _ok("gdn_conv_fwd", load().gdn_conv_fwd(byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens),
                                            int(l2norm_qk), l2_eps, _p(y), _ld(y), _stream(stream)))


def gdn_conv_bwd(shape, x, w, cu_seqlens, dy, dx, dw, ws, l2norm_qk=True, l2_eps=1e-6,
                 stream=None):
    _ok("gdn_conv_bwd", load().gdn_conv_bwd(byref(shape), _p(x), _ld(x), _p(w), _p(cu_seqlens),
                                            int(l2norm_qk), l2_eps, _p(dy), _ld(dy), _p(dx),
                                            _ld(dx), _p(dw), _p(ws), ws.numel() if ws is not None else 0,
                                            _stream(stream)))


def gdn_gate_fwd(shape, a, b, A_log, dt_bias, g, beta, stream=None):
    _ok("gdn_gate_fwd", load().gdn_gate_fwd(byref(shape), _p(a), _p(b), _p(A_log), _p(dt_bias),
                                            _p(g), _p(beta), _stream(stream)))


def gdn_gate_bwd(shape, a, b, A_log, dt_bias, dg, dbeta, da, db, dA_log, ddt_bias, ws,
                 stream=None):
    _ok("gdn_gate_bwd", load().gdn_gate_bwd(byref(shape), _p(a), _p(b), _p(A_log), _p(dt_bias),
                                            _p(dg), _p(dbeta), _p(da), _p(db), _p(dA_log),
                                            _p(ddt_bias), _p(ws), ws.numel() if ws is not None else 0,
                                            _stream(stream)))


def gdn_chunk_fwd(shape, q, k, v, g, beta, scale, S0, S_final, cu_seqlens, o, ws, stream=None):
    _ok("gdn_chunk_fwd", load().gdn_chunk_fwd(byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k),
                                              _ld(v), _p(g), _p(beta), scale, _p(S0), _p(S_final),
                                              _p(cu_seqlens), _p(o), _p(ws), ws.numel(),
                                              _stream(stream)))


def gdn_chunk_bwd(shape, q, k, v, g, beta, scale, S0, cu_seqlens, dout, dS_final, dq, dk, dv, dg,
                  dbeta, dS0, ws, stream=None):
    _ok("gdn_chunk_bwd", load().gdn_chunk_bwd(byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k),
                                              _ld(v), _p(g), _p(beta), scale, _p(S0),
                                              _p(cu_seqlens), _p(dout), _p(dS_final), _p(dq),
                                              _p(dk), _p(dv), _ld(dq), _ld(dk), _ld(dv), _p(dg),
                                              _p(dbeta), _p(dS0), _p(ws), ws.numel(),
                                              _stream(stream)))


def gdn_chunk_prepare(shape, q, k, g, beta, scale, cu_seqlens, ws, stream=None):
    _ok("gdn_chunk_prepare", load().gdn_chunk_prepare(byref(shape), _p(q), _p(k), _ld(q), _ld(k),
                                                      _p(g), _p(beta), scale, _p(cu_seqlens),
                                                      _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_prepare_bwd(shape, q, k, g, beta, scale, cu_seqlens, ws, stream=None):
    _ok("gdn_chunk_prepare_bwd", load().gdn_chunk_prepare_bwd(
        byref(shape), _p(q), _p(k), _ld(q), _ld(k), _p(g), _p(beta), scale, _p(cu_seqlens), _p(ws),
        ws.numel(), _stream(stream)))


def gdn_chunk_fwd_states(shape, q, k, v, scale, S0, S_final, cu_seqlens, o, ws, stream=None):
    _ok("gdn_chunk_fwd_states", load().gdn_chunk_fwd_states(
        byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k), _ld(v), scale, _p(S0), _p(S_final),
        _p(cu_seqlens), _p(o), _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_fwd_states_save(shape, q, k, v, scale, S0, S_final, cu_seqlens, o, ws, stream=None):
    _ok("gdn_chunk_fwd_states_save", load().gdn_chunk_fwd_states_save(
        byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k), _ld(v), scale, _p(S0), _p(S_final),
        _p(cu_seqlens), _p(o), _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_bwd_states(shape, q, k, v, scale, S0, cu_seqlens, ws, stream=None):
    _ok("gdn_chunk_bwd_states", load().gdn_chunk_bwd_states(
        byref(shape), _p(q), _p(k), _p(v), _ld(q), _ld(k), _ld(v), scale, _p(S0), _p(cu_seqlens),
        _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_bwd_reverse(shape, q, k, scale, cu_seqlens, dout, dS_final, dv, dS0, ws, stream=None):
    _ok("gdn_chunk_bwd_reverse", load().gdn_chunk_bwd_reverse(
        byref(shape), _p(q), _p(k), _ld(q), _ld(k), scale, _p(cu_seqlens), _p(dout), _p(dS_final),
        _p(dv), _ld(dv), _p(dS0), _p(ws), ws.numel(), _stream(stream)))


def gdn_chunk_bwd_grads(shape, q, k, beta, scale, cu_seqlens, dout, dv, dq, dk, dg, dbeta, ws,
                        stream=None):
    _ok("gdn_chunk_bwd_grads", load().gdn_chunk_bwd_grads(
        byref(shape), _p(q), _p(k), _ld(q), _ld(k), _p(beta), scale, _p(cu_seqlens), _p(dout),
        _p(dv), _ld(dv), _p(dq), _p(dk), _ld(dq), _ld(dk), _p(dg), _p(dbeta), _p(ws), ws.numel(),
        _stream(stream)))


def gdn_gated_norm_fwd(o, z, w, y, eps=1e-6, act=GDN_ACT_SILU, stream=None):
    dv = o.shape[-1]
    rows = o.numel() // dv
    _ok("gdn_gated_norm_fwd", load().gdn_gated_norm_fwd(rows, dv, _dt(o), _p(o), _p(z), _p(w), eps,
                                                        act, _p(y), _stream(stream)))


def gdn_gated_norm_bwd(o, z, w, dy, dout, dz, dw, ws, eps=1e-6, act=GDN_ACT_SILU, stream=None):
    dv = o.shape[-1]
    rows = o.numel() // dv
    _ok("gdn_gated_norm_bwd", load().gdn_gated_norm_bwd(rows, dv, _dt(o), _p(o), _p(z), _p(w), eps,
                                                        act, _p(dy), _p(dout), _p(dz), _p(dw),
                                                        _p(ws), ws.numel(), _stream(stream)))
