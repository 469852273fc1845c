"""Determinism and out-of-bounds guards on the GPU, through the C ABI.

* Bitwise determinism: the layer core's forward and backward, run twice on
  the same inputs, give bitwise-equal outputs and gradients (there are no
  floating-point atomics; every reduction has a fixed order).  Run at the
  full workload sizes too, where the sequential chunk kernels run long
  enough for an early-released memory wait (a copy consumed before it
  landed) to show as a difference between runs.
* Canary bands: every output and workspace buffer sits between bands of a
  known byte pattern; after every entry point has run, the bands (and the
  inputs) must be unchanged.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_layer_causal_amd import capi as L
from gated_deltanet_layer_causal_amd import inputs as gi
from gated_deltanet_layer_causal_amd.layer import CoreConfig, GDNCore
from tests.gpu_util import DEV, dev, gdn_dtype, torch_dtype

pytestmark = pytest.mark.gpu


def _gpu_inputs(w, seed):
    """The workload's distributions, drawn on the device (no oracle involved)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, C, Hv, d = w.T, w.channels, w.hv, w.d

    def n(shape, std=1.0, dt=torch.float32):
        return (torch.randn(shape, generator=gen, device=DEV) * std).to(dt)

    A = torch.rand(Hv, generator=gen, device=DEV) * (w.A_range[1] - w.A_range[0]) + w.A_range[0]
    if w.seq == "varlen":
        lens = gi.varlen_lengths(np.random.Generator(np.random.PCG64(w.seed)), T)
        cu = torch.from_numpy(gi.cu_from_lengths(lens)).to(DEV)
    else:
        cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    N = cu.numel() - 1
    args = (n((T, C), dt=tdt), n((C, 4), 0.25), n((T, Hv), dt=tdt), n((T, Hv), dt=tdt), torch.log(A),
            torch.zeros(Hv, device=DEV), n((T, Hv, d), dt=tdt), n((d,), 0.1), cu)
    S0 = n((N, Hv, d, d), 0.1) if w.init_state else None
    dST = n((N, Hv, d, d)) if w.final_state else None
    return args, n((T, Hv, d), dt=tdt), S0, dST


def _run_layer(core, args, dy, S0, dST, save_states):
    f = core.forward(*args, S0=S0, want_final=True, save_states=save_states)
    g = core.backward(f, *args, dy, S0=S0, dS_final=dST)
    out = {k: f[k] for k in ("y", "g", "beta", "o", "out", "S_final")}
    out.update(g)
    return out


DET_CASES = {
    "small_varlen": gi.Workload("dv", 0, 2, 6, 128, "bf16", seq="varlen", init_state=True,
                                final_state=True, seed=90),
    "tp4share": gi.WORKLOADS["tp4share"],
    "varlen16k": gi.WORKLOADS["varlen16k"],
    "flash64k": gi.WORKLOADS["flash64k"],
}


@pytest.mark.parametrize("name", list(DET_CASES))
def test_layer_bitwise_deterministic(name):
    w = DET_CASES[name]
    if w.T == 0:
        w = gi.Workload(w.name, 2000, w.hk, w.hv, w.d, w.dtype, seq="varlen", init_state=True,
                        final_state=True, seed=w.seed)
    print(f"[determinism {name}] {w.T} tokens, {w.hk}/{w.hv} heads", flush=True)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    core = GDNCore(CoreConfig(hk=w.hk, hv=w.hv, d=w.d, dtype=tdt), device=DEV)
    args, dy, S0, dST = _gpu_inputs(w, seed=5)
    for save in (True, False):
        r1 = _run_layer(core, args, dy, S0, dST, save)
        r2 = _run_layer(core, args, dy, S0, dST, save)
        torch.cuda.synchronize()
        for k in r1:
            if r1[k] is None:
                continue
            a, b = r1[k], r2[k]
            same = torch.equal(a.view(torch.uint8) if a.dtype != torch.bool else a,
                               b.view(torch.uint8) if b.dtype != torch.bool else b)
            if not same:
                diff = (a.float() - b.float()).abs()
                raise AssertionError(f"{name} save_states={save}: {k} differs between runs "
                                     f"(max |diff| {diff.max().item():.3e}, "
                                     f"{int((diff > 0).sum())} elements)")
        del r1, r2


# ---------------------------------------------------------------------- canaries
BAND = 4096          # bytes of canary on each side of a buffer (keeps 16-byte alignment)
PATTERN = 0xA5


class Guarded:
    """Device buffers with canary bands on both sides."""

    def __init__(self):
        self.bufs = []

    def new(self, name, shape, dtype, fill=None):
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((BAND + max(nbytes, 16) + BAND,), PATTERN, dtype=torch.uint8, device=DEV)
        t = raw[BAND:BAND + nbytes].view(dtype).view(shape)
        if fill is not None:
            t.copy_(fill)
        self.bufs.append((name, raw, nbytes))
        return t

    def check(self):
        bad = []
        for name, raw, nbytes in self.bufs:
            lo = raw[:BAND]
            hi = raw[BAND + max(nbytes, 16):]
            pad = raw[BAND + nbytes:BAND + max(nbytes, 16)]
            for part, t in (("before", lo), ("after", hi), ("padding", pad)):
                if t.numel() and not bool((t == PATTERN).all()):
                    first = int(torch.nonzero(t != PATTERN)[0])
                    bad.append(f"{name}: canary {part} the buffer overwritten at byte {first}")
        assert not bad, "; ".join(bad)


CANARY_CASES = {
    # name: hk, hv, d, dtype, lens, segment length of the state scan
    "bf16_d128": (2, 6, 128, "bf16", [300, 65, 7, 1, 0, 130], 0),
    "bf16_d128_seg": (2, 6, 128, "bf16", [300, 65, 7, 1, 0, 130], 2),
    "bf16_d32": (2, 4, 32, "bf16", [129, 64, 3], 0),
    "bf16_d32_seg": (2, 4, 32, "bf16", [129, 64, 3], 1),
    "fp32_d32": (1, 2, 32, "fp32", [100, 37, 1, 70], 0),
    "fp32_d32_seg": (1, 2, 32, "fp32", [100, 37, 1, 70], 1),
    "fp16_d128_seg": (2, 6, 128, "fp16", [300, 65, 7, 1, 0, 130], 2),
}


@pytest.mark.parametrize("name", list(CANARY_CASES))
def test_every_entry_point_stays_in_bounds(name):
    hk, hv, d, dt, lens, seg = CANARY_CASES[name]
    w = gi.Workload(name, sum(lens), hk, hv, d, dt, seq="varlen", init_state=True,
                    final_state=True, seed=91)
    inp = gi.make_inputs(w, seqlens=lens, A_range=(0.02, 0.3))
    tdt = torch_dtype(dt)
    T, N, C = inp["T"], inp["N"], w.channels
    sh = L.make_shape(N, T, hk, hv, d, gdn_dtype(dt), seg)
    G = Guarded()
    # inputs (checked afterwards to be unchanged)
    x = G.new("x", (T, C), tdt, dev(inp["x"], tdt))
    wc = G.new("w_conv", (C, 4), torch.float32, dev(inp["w_conv"]))
    cu = G.new("cu_seqlens", (N + 1,), torch.int32, torch.from_numpy(inp["cu_seqlens"]).to(DEV))
    a = G.new("a", (T, hv), tdt, dev(inp["a"], tdt))
    b = G.new("b", (T, hv), tdt, dev(inp["b"], tdt))
    Al = G.new("A_log", (hv,), torch.float32, dev(inp["A_log"]))
    dtb = G.new("dt_bias", (hv,), torch.float32, dev(inp["dt_bias"]))
    z = G.new("z", (T, hv, d), tdt, dev(inp["z"], tdt))
    wn = G.new("w_norm", (d,), torch.float32, dev(inp["w_norm"]))
    S0 = G.new("S0", (N, hv, d, d), torch.float32, dev(inp["S0"]))
    dST = G.new("dS_T", (N, hv, d, d), torch.float32, dev(inp["dS_T"]))
    dy = G.new("dy", (T, hv, d), tdt, dev(inp["dy"], tdt))
    inputs = {k: t.clone() for k, t in (("x", x), ("w_conv", wc), ("cu", cu), ("a", a), ("b", b),
                                        ("A_log", Al), ("dt_bias", dtb), ("z", z), ("w_norm", wn),
                                        ("S0", S0), ("dS_T", dST), ("dy", dy))}
    scale = d ** -0.5
    ws_small = G.new("ws", (max(L.gdn_conv_bwd_workspace(sh), L.gdn_gate_bwd_workspace(sh),
                                L.gdn_gated_norm_bwd_workspace(T * hv, d), 16),), torch.uint8)
    # forward
    y = G.new("y", (T, C), tdt)
    L.gdn_conv_fwd(sh, x, wc, cu, y)
    g = G.new("g", (T, hv), torch.float32)
    beta = G.new("beta", (T, hv), torch.float32)
    L.gdn_gate_fwd(sh, a, b, Al, dtb, g, beta)
    q, k, v = y[:, : hk * d], y[:, hk * d: 2 * hk * d], y[:, 2 * hk * d:]
    dout = G.new("dout_chunk", (T, hv, d), tdt, dy)
    outs = {}
    for flow in ("composite", "saved"):
        wsc = G.new(f"chunk_ws_{flow}", (L.gdn_chunk_bwd_workspace(sh),), torch.uint8)
        o = G.new(f"o_{flow}", (T, hv, d), tdt)
        Sf = G.new(f"S_final_{flow}", (N, hv, d, d), torch.float32)
        dyc = G.new(f"dy_chunk_{flow}", (T, C), tdt)
        dq, dk, dv = dyc[:, : hk * d], dyc[:, hk * d: 2 * hk * d], dyc[:, 2 * hk * d:]
        dg = G.new(f"dg_{flow}", (T, hv), torch.float32)
        db = G.new(f"dbeta_{flow}", (T, hv), torch.float32)
        dS0 = G.new(f"dS0_{flow}", (N, hv, d, d), torch.float32)
        if flow == "composite":
            wsf = G.new("chunk_ws_fwd", (L.gdn_chunk_fwd_workspace(sh),), torch.uint8)
            L.gdn_chunk_fwd(sh, q, k, v, g, beta, scale, S0, Sf, cu, o, wsf)
            L.gdn_chunk_bwd(sh, q, k, v, g, beta, scale, S0, cu, dout, dST, dq, dk, dv, dg, db,
                            dS0, wsc)
        else:
            L.gdn_chunk_prepare_bwd(sh, q, k, g, beta, scale, cu, wsc)
            L.gdn_chunk_fwd_states_save(sh, q, k, v, scale, S0, Sf, cu, o, wsc)
            L.gdn_chunk_bwd_reverse(sh, q, k, scale, cu, dout, dST, dv, dS0, wsc)
            L.gdn_chunk_bwd_grads(sh, q, k, beta, scale, cu, dout, dv, dq, dk, dg, db, wsc)
        outs[flow] = o
    ynorm = G.new("y_norm", (T, hv, d), tdt)
    L.gdn_gated_norm_fwd(outs["saved"], z, wn, ynorm)
    do = G.new("do", (T, hv, d), tdt)
    dz = G.new("dz", (T, hv, d), tdt)
    dwn = G.new("dw_norm", (d,), torch.float32)
    L.gdn_gated_norm_bwd(outs["saved"], z, wn, dy, do, dz, dwn, ws_small)
    dgg = G.new("dg_in", (T, hv), torch.float32, g)
    dbb = G.new("dbeta_in", (T, hv), torch.float32, beta)
    da = G.new("da", (T, hv), tdt)
    dbo = G.new("db", (T, hv), tdt)
    dAl = G.new("dA_log", (hv,), torch.float32)
    ddt = G.new("ddt_bias", (hv,), torch.float32)
    L.gdn_gate_bwd(sh, a, b, Al, dtb, dgg, dbb, da, dbo, dAl, ddt, ws_small)
    dyconv = G.new("dy_conv", (T, C), tdt, y)
    dx = G.new("dx", (T, C), tdt)
    dwc = G.new("dw_conv", (C, 4), torch.float32)
    L.gdn_conv_bwd(sh, x, wc, cu, dyconv, dx, dwc, ws_small)
    torch.cuda.synchronize()
    G.check()
    now = {"x": x, "w_conv": wc, "cu": cu, "a": a, "b": b, "A_log": Al, "dt_bias": dtb, "z": z,
           "w_norm": wn, "S0": S0, "dS_T": dST, "dy": dy}
    for kname, t in inputs.items():
        assert torch.equal(t, now[kname]), f"input {kname} was written"
