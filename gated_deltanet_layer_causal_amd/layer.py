"""Gated DeltaNet layer core on top of libgdn: conv -> gate -> chunked gated
delta rule -> gated norm, forward and backward.

This module only allocates outputs/workspace with torch and calls the C ABI
in order; every step of the computation runs in the HIP kernels.

Token tensors: x [T, C] (q | k | v channels), z [T, Hv, d], output [T, Hv, d].
"""
from __future__ import annotations

import contextlib
import dataclasses
from typing import Optional

import torch

from . import capi as L


@dataclasses.dataclass
class CoreConfig:
    hk: int
    hv: int
    d: int
    dtype: torch.dtype = torch.bfloat16
    scale: Optional[float] = None        # default d ** -0.5
    act: int = L.GDN_ACT_SILU            # output-gate activation
    l2_eps: float = 1e-6
    norm_eps: float = 1e-6
    seg_chunks: int = 0                  # segment-parallel state scan (0: the library decides)
    check_cu_seqlens: bool = False       # debug: check the cu_seqlens contract (synchronises)

    @property
    def channels(self):
        return 2 * self.hk * self.d + self.hv * self.d

    @property
    def q_scale(self):
        return self.d ** -0.5 if self.scale is None else self.scale


@contextlib.contextmanager
def _timed(timer, name):
    """Optional hook (e.g. HIP events) around one C-ABI call."""
    if timer is not None:
        timer(name, "begin")
    yield
    if timer is not None:
        timer(name, "end")


class GDNCore:
    """Runs the layer core's forward and backward for one configuration.

    Training flow (save_states=True, the default): the forward runs the
    backward-mode chunk preparation and the state pass that also stores the
    chunk-start states, R and Delta in a per-call chunk workspace, which the
    backward then consumes (reverse pass + chunk gradients only).  With
    save_states=False the forward keeps only its outputs and the backward
    recomputes the preparation and the states."""

    def __init__(self, cfg: CoreConfig, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self._ws = None        # conv / gate / norm scratch
        self._ws_chunk = None  # chunk scratch of calls that do not save states
        L.load()

    def shape(self, T: int, n_seq: int) -> L.Shape:
        c = self.cfg
        return L.make_shape(n_seq, T, c.hk, c.hv, c.d, c.dtype, c.seg_chunks)

    def workspace(self, shape: L.Shape, rows: int) -> torch.Tensor:
        need = max(L.gdn_conv_bwd_workspace(shape), L.gdn_gate_bwd_workspace(shape),
                   L.gdn_gated_norm_bwd_workspace(rows, self.cfg.d), 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def chunk_workspace(self, shape: L.Shape, fresh: bool) -> torch.Tensor:
        need = L.gdn_chunk_bwd_workspace(shape)
        if fresh:
            return torch.empty(need, dtype=torch.uint8, device=self.device)
        if self._ws_chunk is None or self._ws_chunk.numel() < need:
            self._ws_chunk = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws_chunk

    def split(self, y):
        c = self.cfg
        q = y[:, : c.hk * c.d]
        k = y[:, c.hk * c.d: 2 * c.hk * c.d]
        v = y[:, 2 * c.hk * c.d:]
        return q, k, v

    def forward(self, x, w_conv, a, b, A_log, dt_bias, z, w_norm, cu_seqlens, S0=None,
                want_final=False, timer=None, save_states=True, conv_state=None,
                want_conv_state=False):
        """conv_state [n_seq, 3, C] (optional): the carried conv state, the
        three input rows before each sequence; with want_conv_state the
        returned dict holds the final one under "conv_state_out" (the last
        three input rows of each sequence), so that a later call continues
        the sequences (feed S_final and conv_state_out back in)."""
        c = self.cfg
        T = x.shape[0]
        n_seq = cu_seqlens.numel() - 1
        sh = self.shape(T, n_seq)
        if c.check_cu_seqlens:
            self.check_cu_seqlens(sh, cu_seqlens)
        ws = self.workspace(sh, T * c.hv)
        wc = self.chunk_workspace(sh, fresh=save_states)
        dev, dt = x.device, c.dtype
        y = torch.empty((T, c.channels), dtype=dt, device=dev)
        cs_out = (torch.empty((n_seq, 3, c.channels), dtype=dt, device=dev) if want_conv_state
                  else None)
        with _timed(timer, "conv_fwd"):
            if conv_state is None and cs_out is None:
                L.gdn_conv_fwd(sh, x, w_conv, cu_seqlens, y, True, c.l2_eps)
            else:
                L.gdn_conv_fwd_state(sh, x, w_conv, cu_seqlens, y, conv_state, cs_out, True,
                                     c.l2_eps)
        g = torch.empty((T, c.hv), dtype=torch.float32, device=dev)
        beta = torch.empty_like(g)
        with _timed(timer, "gate_fwd"):
            L.gdn_gate_fwd(sh, a, b, A_log, dt_bias, g, beta)
        q, k, v = self.split(y)
        o = torch.empty((T, c.hv, c.d), dtype=dt, device=dev)
        Sf = torch.empty((n_seq, c.hv, c.d, c.d), dtype=torch.float32, device=dev) if want_final else None
        if save_states:
            with _timed(timer, "chunk_prepare"):
                L.gdn_chunk_prepare_bwd(sh, q, k, g, beta, c.q_scale, cu_seqlens, wc)
            with _timed(timer, "chunk_fwd_states"):
                L.gdn_chunk_fwd_states_save(sh, q, k, v, c.q_scale, S0, Sf, cu_seqlens, o, wc)
        else:
            with _timed(timer, "chunk_prepare"):
                L.gdn_chunk_prepare(sh, q, k, g, beta, c.q_scale, cu_seqlens, wc)
            with _timed(timer, "chunk_fwd_states"):
                L.gdn_chunk_fwd_states(sh, q, k, v, c.q_scale, S0, Sf, cu_seqlens, o, wc)
        out = torch.empty_like(o)
        with _timed(timer, "norm_fwd"):
            L.gdn_gated_norm_fwd(o, z, w_norm, out, c.norm_eps, c.act)
        saved = {"y": y, "g": g, "beta": beta, "o": o, "out": out, "S_final": Sf,
                 "conv_state_out": cs_out}
        if save_states:
            saved["chunk_ws"] = wc
        return saved

    def check_cu_seqlens(self, sh, cu_seqlens):
        """Runs gdn_check_cu_seqlens and raises ValueError naming each broken
        part of the contract (this waits for the stream)."""
        out = torch.empty(1, dtype=torch.int32, device=cu_seqlens.device)
        L.gdn_check_cu_seqlens(sh, cu_seqlens, out)
        bad = int(out.item())
        if bad:
            why = [msg for bit, msg in ((L.CU_BAD_START, "cu_seqlens[0] != 0"),
                                        (L.CU_BAD_END, "cu_seqlens[-1] != the token count"),
                                        (L.CU_DECREASING, "cu_seqlens decreases"))
                   if bad & bit]
            raise ValueError("invalid cu_seqlens: " + "; ".join(why))

    def backward(self, saved, x, w_conv, a, b, A_log, dt_bias, z, w_norm, cu_seqlens, dout,
                 S0=None, dS_final=None, timer=None, conv_state=None, d_conv_state=None):
        """conv_state: the forward's; d_conv_state: the gradient of its final
        conv state.  With either, the result holds "d_conv_state" (the
        gradient of the carried conv state that came in)."""
        c = self.cfg
        T = x.shape[0]
        n_seq = cu_seqlens.numel() - 1
        sh = self.shape(T, n_seq)
        ws = self.workspace(sh, T * c.hv)
        dev, dt = x.device, c.dtype
        do = torch.empty((T, c.hv, c.d), dtype=dt, device=dev)
        dz = torch.empty_like(do)
        dw_norm = torch.empty(c.d, dtype=torch.float32, device=dev)
        with _timed(timer, "norm_bwd"):
            L.gdn_gated_norm_bwd(saved["o"], z, w_norm, dout, do, dz, dw_norm, ws, c.norm_eps,
                                 c.act)
        dy = torch.empty((T, c.channels), dtype=dt, device=dev)
        dq, dk, dv = self.split(dy)
        dg = torch.empty((T, c.hv), dtype=torch.float32, device=dev)
        dbeta = torch.empty_like(dg)
        dS0 = torch.empty((n_seq, c.hv, c.d, c.d), dtype=torch.float32, device=dev)
        q, k, v = self.split(saved["y"])
        wc = saved.get("chunk_ws")
        if wc is None:
            wc = self.chunk_workspace(sh, fresh=False)
            with _timed(timer, "chunk_prepare_b"):
                L.gdn_chunk_prepare_bwd(sh, q, k, saved["g"], saved["beta"], c.q_scale, cu_seqlens,
                                        wc)
            with _timed(timer, "chunk_bwd_states"):
                L.gdn_chunk_bwd_states(sh, q, k, v, c.q_scale, S0, cu_seqlens, wc)
        with _timed(timer, "chunk_bwd_reverse"):
            L.gdn_chunk_bwd_reverse(sh, q, k, c.q_scale, cu_seqlens, do, dS_final, dv, dS0, wc)
        with _timed(timer, "chunk_bwd_grads"):
            L.gdn_chunk_bwd_grads(sh, q, k, saved["beta"], c.q_scale, cu_seqlens, do, dv, dq, dk, dg,
                                  dbeta, wc)
        da = torch.empty((T, c.hv), dtype=dt, device=dev)
        db = torch.empty_like(da)
        dA_log = torch.empty(c.hv, dtype=torch.float32, device=dev)
        ddt = torch.empty_like(dA_log)
        with _timed(timer, "gate_bwd"):
            L.gdn_gate_bwd(sh, a, b, A_log, dt_bias, dg, dbeta, da, db, dA_log, ddt, ws)
        dx = torch.empty((T, c.channels), dtype=dt, device=dev)
        dw_conv = torch.empty((c.channels, 4), dtype=torch.float32, device=dev)
        dcs_in = None
        with _timed(timer, "conv_bwd"):
            if conv_state is None and d_conv_state is None:
                L.gdn_conv_bwd(sh, x, w_conv, cu_seqlens, dy, dx, dw_conv, ws, True, c.l2_eps)
            else:
                dcs_in = torch.empty((n_seq, 3, c.channels), dtype=dt, device=dev)
                L.gdn_conv_bwd_state(sh, x, w_conv, cu_seqlens, dy, dx, dw_conv, ws, conv_state,
                                     d_conv_state, dcs_in, True, c.l2_eps)
        return {"do": do, "dz": dz, "dw_norm": dw_norm, "dy_conv": dy, "dg": dg, "dbeta": dbeta,
                "dS0": dS0, "da": da, "db": db, "dA_log": dA_log, "ddt_bias": ddt, "dx": dx,
                "dw_conv": dw_conv, "d_conv_state": dcs_in}


class GDNLayer:
    """The layer with its projections: hidden states X [T, H] -> in_proj ->
    GDNCore -> out_proj -> Y [T, H], forward and backward.

    The projections are plain GEMMs, left to the library (torch.matmul, which
    runs hipBLASLt on ROCm); everything between them is GDNCore, i.e. libgdn.
    in_proj is three products so that each core input is contiguous:
    x = X W_x^T (q | k | v channels), z = X W_z^T and [a | b] = X [W_a | W_b]^T
    (a and b, hv columns each, are then copied apart);
    out_proj is Y = out W_out^T.  Weights are held in both layouts, [out, in]
    and [in, out], and each product takes the operand order that the library
    runs fastest (measured at 65536 tokens, hidden 2560, bf16): the forward
    as X (W)^T and dX as G (W^T)^T, i.e. the right operand a transposed view,
    and dW as (X^T G)^T; 19.7 ms for the layer's fifteen products against
    21.5 ms with contiguous right operands."""

    NAMES = ("x", "z", "a", "b", "out")

    def __init__(self, cfg: CoreConfig, hidden: int, weights: dict, device="cuda"):
        """weights: name -> [out, in] tensors (the nn.Linear convention)."""
        self.core = GDNCore(cfg, device)
        self.cfg = cfg
        self.hidden = hidden
        self.W = {k: weights[k].contiguous() for k in self.NAMES}        # [out, in]
        # a and b (hv outputs each) as one product, so that X is read once for
        # both and the gradients make one pass each
        self.W["ab"] = torch.cat([self.W["a"], self.W["b"]], 0)
        self.Wt = {k: w.t().contiguous() for k, w in self.W.items()}      # [in, out]

    def forward(self, X, w_conv, A_log, dt_bias, w_norm, cu_seqlens, S0=None, want_final=False,
                timer=None):
        c = self.cfg
        T = X.shape[0]
        with _timed(timer, "in_proj"):
            x = X @ self.W["x"].t()
            z = (X @ self.W["z"].t()).view(T, c.hv, c.d)
            ab = X @ self.W["ab"].t()
            a = ab[:, :c.hv].contiguous()
            b = ab[:, c.hv:].contiguous()
        f = self.core.forward(x, w_conv, a, b, A_log, dt_bias, z, w_norm, cu_seqlens, S0=S0,
                              want_final=want_final, timer=timer)
        out = f["out"].view(T, c.hv * c.d)
        with _timed(timer, "out_proj"):
            Y = out @ self.W["out"].t()
        f.update(x=x, z=z, a=a, b=b, Y=Y)
        return f

    def backward(self, saved, X, w_conv, A_log, dt_bias, w_norm, cu_seqlens, dY, S0=None,
                 dS_final=None, timer=None):
        c = self.cfg
        T = X.shape[0]
        with _timed(timer, "out_proj_bwd"):
            dout = (dY @ self.Wt["out"].t()).view(T, c.hv, c.d)
            dW_out = (saved["out"].view(T, c.hv * c.d).t() @ dY).t()
        g = self.core.backward(saved, saved["x"], w_conv, saved["a"], saved["b"], A_log, dt_bias,
                               saved["z"], w_norm, cu_seqlens, dout, S0=S0, dS_final=dS_final,
                               timer=timer)
        with _timed(timer, "in_proj_bwd"):
            gz = g["dz"].view(T, c.hv * c.d)
            dX = g["dx"] @ self.Wt["x"].t()
            dX.addmm_(gz, self.Wt["z"].t())
            dab = torch.cat([g["da"], g["db"]], 1)
            dX.addmm_(dab, self.Wt["ab"].t())
            Xt = X.t()
            dW_ab = (Xt @ dab).t()
            dW = {"x": (Xt @ g["dx"]).t(), "z": (Xt @ gz).t(), "a": dW_ab[:c.hv], "b": dW_ab[c.hv:],
                  "out": dW_out}
        g.update(dX=dX, dW=dW, dout=dout)
        return g
