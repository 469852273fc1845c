"""Per-op GPU parity against the CPU oracle (run through the C ABI).

Every op is fed bit-identical inputs on both sides: inputs come from the
seeded generator, or from an earlier oracle op rounded to the storage dtype.
Shapes are small enough for the oracle yet span several 64-token chunks,
ragged tails, a length-1 sequence and grouped value heads.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_layer_causal_amd import inputs as gi
from gated_deltanet_layer_causal_amd import capi as L
from tests.gpu_util import (DEV, FWD_TOL_BF16, GRAD_TOL_BF16, TOL_FP32, assert_close, dev, host,
                            rel_err)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (hk, hv, d, dtype, lens, A_range, S0/final)
    "fp32_tiny": (1, 2, 32, "fp32", [64], (1.0, 16.0), False),
    "fp32_ragged": (1, 2, 32, "fp32", [100, 37, 1, 70], (0.02, 0.2), True),
    "bf16_g2_mild": (2, 4, 128, "bf16", [150, 64, 1, 90], (0.01, 0.1), True),
    "bf16_g3_strong": (2, 6, 128, "bf16", [200, 7, 130], (1.0, 16.0), False),
    "bf16_d32": (2, 4, 32, "bf16", [129, 64], (0.05, 0.5), True),
    "fp16_g2_mild": (2, 4, 128, "fp16", [150, 64, 1, 90], (0.01, 0.1), True),
    "fp16_d32": (2, 4, 32, "fp16", [129, 64, 2], (0.05, 0.5), True),
}
# conv only: 3 k-heads of 128 put the end of the q and k channels (768) inside
# the second 512-channel block, so one launch runs every L2 mode of the conv
# kernels (all lanes normalise, some do, none do)
CONV_EXTRA = {
    "bf16_l2mix": (3, 3, 128, "bf16", [150, 3, 70], (0.01, 0.1), False),
}


def _tol(dtype, grad=False):
    if dtype == "fp32":
        return TOL_FP32
    return GRAD_TOL_BF16 if grad else FWD_TOL_BF16


def _rnd(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    r = gi.round_to(dtype)
    return a if r is None else r(a)


def _tdt(dtype):
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]


def _gdt(dtype):
    return {"bf16": L.GDN_BF16, "fp16": L.GDN_FP16, "fp32": L.GDN_FP32}[dtype]


def _case(name, seed=7):
    hk, hv, d, dtype, lens, A_range, state = CASES[name] if name in CASES else CONV_EXTRA[name]
    w = gi.Workload(name, sum(lens), hk, hv, d, dtype, seq="varlen", init_state=state,
                    final_state=state, seed=seed)
    inp = gi.make_inputs(w, seqlens=lens, A_range=A_range)
    return w, inp


def _shape(w, inp):
    return L.make_shape(inp["N"], inp["T"], w.hk, w.hv, w.d, _gdt(w.dtype))


# ------------------------------------------------------------------ conv
@pytest.mark.parametrize("name", list(CASES) + list(CONV_EXTRA))
def test_conv_fwd_bwd(name):
    w, inp = _case(name)
    dt = w.dtype
    cu = inp["cu_seqlens"]
    n_l2 = 2 * w.hk * w.d
    y_ref = oracle.conv_fwd(inp["x"], inp["w_conv"], cu, n_l2, w.d)
    rng = np.random.default_rng(3)
    dy = _rnd(rng.standard_normal(y_ref.shape), dt)
    dx_ref, dw_ref = oracle.conv_bwd(inp["x"], inp["w_conv"], cu, n_l2, w.d, dy)

    sh = _shape(w, inp)
    x = dev(inp["x"], _tdt(dt))
    wc = dev(inp["w_conv"])
    cut = torch.from_numpy(cu).to(DEV)
    y = torch.empty_like(x)
    L.gdn_conv_fwd(sh, x, wc, cut, y)
    dyt = dev(dy, _tdt(dt))
    dx = torch.empty_like(x)
    dw = torch.empty_like(wc)
    ws = torch.empty(max(L.gdn_conv_bwd_workspace(sh), 16), dtype=torch.uint8, device=DEV)
    L.gdn_conv_bwd(sh, x, wc, cut, dyt, dx, dw, ws)
    torch.cuda.synchronize()
    assert_close("y", host(y), y_ref, _tol(dt))
    assert_close("dx", host(dx), dx_ref, _tol(dt, True))
    assert_close("dw", host(dw), dw_ref, _tol(dt, True))


# ------------------------------------------------------------------ gate
@pytest.mark.parametrize("name", ["fp32_tiny", "bf16_g3_strong", "fp16_g2_mild"])
def test_gate_fwd_bwd(name):
    w, inp = _case(name)
    dt = w.dtype
    g_ref, b_ref = oracle.gate_fwd(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    rng = np.random.default_rng(4)
    dg = rng.standard_normal(g_ref.shape).astype(np.float32)
    dbeta = rng.standard_normal(g_ref.shape).astype(np.float32)
    ref = oracle.gate_bwd(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], dg, dbeta)
    sh = _shape(w, inp)
    a, b = dev(inp["a"], _tdt(dt)), dev(inp["b"], _tdt(dt))
    Al, dtb = dev(inp["A_log"]), dev(inp["dt_bias"])
    g = torch.empty(a.shape, dtype=torch.float32, device=DEV)
    beta = torch.empty_like(g)
    L.gdn_gate_fwd(sh, a, b, Al, dtb, g, beta)
    da, db = torch.empty_like(a), torch.empty_like(b)
    dAl, ddt = torch.empty_like(Al), torch.empty_like(dtb)
    ws = torch.empty(L.gdn_gate_bwd_workspace(sh), dtype=torch.uint8, device=DEV)
    L.gdn_gate_bwd(sh, a, b, Al, dtb, dev(dg), dev(dbeta), da, db, dAl, ddt, ws)
    torch.cuda.synchronize()
    tol = TOL_FP32 if dt == "fp32" else FWD_TOL_BF16
    assert_close("g", host(g), g_ref, TOL_FP32)
    assert_close("beta", host(beta), b_ref, TOL_FP32)
    for nm, got, r in (("da", da, ref[0]), ("db", db, ref[1]), ("dA_log", dAl, ref[2]),
                       ("ddt_bias", ddt, ref[3])):
        assert_close(nm, host(got), r, tol if nm in ("da", "db") else TOL_FP32 * 10)


# ------------------------------------------------------------------ gated norm
@pytest.mark.parametrize("name", ["fp32_tiny", "bf16_g2_mild", "bf16_d32", "fp16_g2_mild", "fp16_d32"])
@pytest.mark.parametrize("act", [L.GDN_ACT_SILU, L.GDN_ACT_SIGMOID])
def test_gated_norm_fwd_bwd(name, act):
    w, inp = _case(name)
    dt = w.dtype
    rng = np.random.default_rng(5)
    o = _rnd(rng.standard_normal(inp["z"].shape), dt)
    y_ref = oracle.norm_fwd(o, inp["z"], inp["w_norm"], act)
    do_ref, dz_ref, dw_ref = oracle.norm_bwd(o, inp["z"], inp["w_norm"], inp["dy"], act)
    ot, zt = dev(o, _tdt(dt)), dev(inp["z"], _tdt(dt))
    wn = dev(inp["w_norm"])
    y = torch.empty_like(ot)
    L.gdn_gated_norm_fwd(ot, zt, wn, y, act=act)
    dyt = dev(inp["dy"], _tdt(dt))
    do, dz, dw = torch.empty_like(ot), torch.empty_like(ot), torch.empty_like(wn)
    ws = torch.empty(L.gdn_gated_norm_bwd_workspace(o.size // w.d, w.d), dtype=torch.uint8, device=DEV)
    L.gdn_gated_norm_bwd(ot, zt, wn, dyt, do, dz, dw, ws, act=act)
    torch.cuda.synchronize()
    assert_close("y", host(y), y_ref, _tol(dt))
    assert_close("do", host(do), do_ref, _tol(dt, True))
    assert_close("dz", host(dz), dz_ref, _tol(dt, True))
    assert_close("dw", host(dw), dw_ref, _tol(dt, True))


# ------------------------------------------------------------------ chunked delta rule
def _delta_inputs(name, seed=7):
    w, inp = _case(name, seed)
    dt = w.dtype
    cu = inp["cu_seqlens"]
    y = _rnd(oracle.conv_fwd(inp["x"], inp["w_conv"], cu, 2 * w.hk * w.d, w.d), dt)
    g, beta = oracle.gate_fwd(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    g, beta = g.astype(np.float32), beta.astype(np.float32)
    return w, inp, y, g, beta


@pytest.mark.parametrize("name", list(CASES))
def test_chunk_fwd_bwd(name):
    """Both chunk flows, each with one sequential pass per sequence (seg 0 at
    these sizes) and with the segment-parallel scan forced to segments of 1
    and 3 chunks (so sequences of several chunks combine several segments,
    and short ones have one)."""
    from tests.gpu_util import FLOWS, run_chunk
    w, inp, y, g, beta = _delta_inputs(name)
    dt, cu, hk, hv, d = w.dtype, inp["cu_seqlens"], w.hk, w.hv, w.d
    scale = d ** -0.5
    T = inp["T"]
    q, k, v = gi.split_qkv(y, hk, hv, d)
    S0 = inp["S0"]
    o_ref, Sf_ref = oracle.delta_fwd(q, k, v, g, beta, cu, scale, S0)
    rng = np.random.default_rng(6)
    dout = _rnd(rng.standard_normal(o_ref.shape), dt)
    dSf = inp["dS_T"]
    ref = oracle.delta_bwd(q, k, v, g, beta, cu, scale, dout, S0, dSf)
    refs = {"o": o_ref, "S_final": Sf_ref, "dq": ref[0], "dk": ref[1], "dv": ref[2], "dg": ref[3],
            "dbeta": ref[4], "dS0": ref[5]}

    yt = dev(y, _tdt(dt))
    qt, kt, vt = yt[:, : hk * d], yt[:, hk * d: 2 * hk * d], yt[:, 2 * hk * d:]
    gt, bt = dev(g), dev(beta)
    cut = torch.from_numpy(cu).to(DEV)
    S0t = dev(S0) if S0 is not None else None
    dSft = dev(dSf) if dSf is not None else None
    dot = dev(dout, _tdt(dt))
    for seg in (0, 1, 3):
        sh = L.make_shape(inp["N"], T, hk, hv, d, _gdt(dt), seg)
        ws = torch.empty(L.gdn_chunk_bwd_workspace(sh), dtype=torch.uint8, device=DEV)
        for flow in FLOWS:
            r = run_chunk(flow, sh, qt, kt, vt, gt, bt, scale, S0t, cut, dot, dSft, ws)
            torch.cuda.synchronize()
            got = {"o": host(r["o"]), "S_final": host(r["S_final"]),
                   "dq": host(r["dq"]).reshape(T, hk, d), "dk": host(r["dk"]).reshape(T, hk, d),
                   "dv": host(r["dv"]).reshape(T, hv, d), "dg": host(r["dg"]),
                   "dbeta": host(r["dbeta"]), "dS0": host(r["dS0"])}
            report = {nm: rel_err(got[nm], refs[nm]) for nm in refs}
            print(name, flow, f"seg={seg}", " ".join(f"{k}={v:.2e}" for k, v in report.items()),
                  flush=True)
            for nm in refs:
                assert_close(f"{nm} ({flow}, seg {seg})", got[nm], refs[nm],
                             _tol(dt, nm not in ("o", "S_final")))


# ------------------------------------------------------------------ chunk table (integer)
def _align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("seg", [0, 1, 3], ids=["seq", "seg1", "seg3"])
@pytest.mark.parametrize("lens", [[70, 0, 64, 0, 5, 1, 128, 129], [3, 0], [1], [0, 0, 3],
                                  [64] * 7 + [65], [64 * 7]],
                         ids=["mixed", "trailing_empty", "one", "leading_empty", "exact_chunks",
                              "one_long"])
def test_chunk_table_exact(lens, seg):
    """The tables the preparation builds from cu_seqlens, bit-exact against
    plain counts.  At the head of the workspace: int32 [n_seq + 1], entry n =
    number of 64-token chunks of sequences 0 .. n-1.  Then (each region
    256-byte aligned) the spans the sequential passes walk, int32 [.][4] =
    (first chunk, end chunk, first token, end token of the sequence): one per
    sequence, or with the segmented scan ceil(chunks / seg) per sequence
    (none for an empty sequence); then int32 [n_seq + 1], the first span of
    each sequence."""
    hk, hv, d = 1, 2, 32
    cu = gi.cu_from_lengths(lens)
    T, N = int(cu[-1]), len(lens)
    sh = L.make_shape(N, T, hk, hv, d, L.GDN_BF16, seg)
    y = torch.zeros((T, 4 * d), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((T, hv), dtype=torch.float32, device=DEV)
    ws = torch.full((L.gdn_chunk_fwd_workspace(sh),), 0x5A, dtype=torch.uint8, device=DEV)
    L.gdn_chunk_prepare(sh, y[:, :d], y[:, d:2 * d], g, g, 1.0, torch.from_numpy(cu).to(DEV), ws)
    torch.cuda.synchronize()
    raw = ws.cpu()
    want = np.zeros(N + 1, dtype=np.int32)
    for n, ln in enumerate(lens):
        want[n + 1] = want[n] + (ln + 63) // 64
    np.testing.assert_array_equal(raw[: 4 * (N + 1)].view(torch.int32).numpy(), want)
    spans, segb = [], [0]
    for n, ln in enumerate(lens):
        nc = (ln + 63) // 64
        if seg == 0:
            spans.append((want[n], want[n + 1], cu[n], cu[n + 1]))
        else:
            for c0 in range(0, nc, seg):
                spans.append((want[n] + c0, want[n] + min(c0 + seg, nc), cu[n] + 64 * c0, cu[n + 1]))
        segb.append(len(spans))
    nt_max = T // 64 + N
    nspan_max = nt_max // seg + N + 1 if seg else N
    assert len(spans) <= nspan_max
    o_sp = _align256(4 * (N + 1))
    o_sb = o_sp + _align256(16 * nspan_max)
    got_sp = raw[o_sp: o_sp + 16 * len(spans)].view(torch.int32).numpy().reshape(-1, 4)
    np.testing.assert_array_equal(got_sp, np.array(spans, dtype=np.int32).reshape(-1, 4))
    np.testing.assert_array_equal(raw[o_sb: o_sb + 4 * (N + 1)].view(torch.int32).numpy(),
                                  np.array(segb, dtype=np.int32))


# ------------------------------------------------------------------ fp16 operand range
@pytest.mark.parametrize("cu,total,want", [
    ([0, 70, 70, 134, 200], 200, 0),
    ([0, 0, 0], 0, 0),
    ([1, 70, 200], 200, L.CU_BAD_START),
    ([0, 70, 199], 200, L.CU_BAD_END),
    ([0, 70, 60, 200], 200, L.CU_DECREASING),
    ([5, 3, 2], 9, L.CU_BAD_START | L.CU_BAD_END | L.CU_DECREASING),
    (list(range(0, 4001, 4)) + [3999], 3999, L.CU_DECREASING),   # past one block of 256 threads
])
def test_check_cu_seqlens(cu, total, want):
    """gdn_check_cu_seqlens reports each broken part of the cu_seqlens
    contract (bit-exact mask), and nothing for valid tables (empty
    sequences included)."""
    n_seq = len(cu) - 1
    print(f"[check_cu_seqlens] n_seq={n_seq} T={total}", flush=True)
    sh = L.make_shape(n_seq, total, 1, 2, 128, L.GDN_BF16)
    cut = torch.tensor(cu, dtype=torch.int32, device=DEV)
    out = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    L.gdn_check_cu_seqlens(sh, cut, out)
    torch.cuda.synchronize()
    assert int(out.item()) == want


def test_layer_refuses_bad_cu_seqlens_when_checking():
    """CoreConfig(check_cu_seqlens=True): a broken table raises before any
    other call is launched; a valid one runs."""
    from gated_deltanet_layer_causal_amd.layer import CoreConfig, GDNCore
    core = GDNCore(CoreConfig(hk=1, hv=2, d=32, dtype=torch.bfloat16, check_cu_seqlens=True),
                   device=DEV)
    T, C = 100, core.cfg.channels
    x = torch.randn(T, C, device=DEV).to(torch.bfloat16)
    wc = torch.randn(C, 4, device=DEV) * 0.5
    a, b = torch.randn(T, 2, device=DEV).to(torch.bfloat16), torch.randn(T, 2, device=DEV).to(torch.bfloat16)
    A_log, dtb = torch.zeros(2, device=DEV), torch.zeros(2, device=DEV)
    z = torch.randn(T, 2, 32, device=DEV).to(torch.bfloat16)
    wn = torch.zeros(32, device=DEV)
    good = torch.tensor([0, 40, 100], dtype=torch.int32, device=DEV)
    core.forward(x, wc, a, b, A_log, dtb, z, wn, good)
    bad = torch.tensor([0, 60, 40, 100], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="decreases"):
        core.forward(x, wc, a, b, A_log, dtb, z, wn, bad)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("flow", ["composite", "saved"])
def test_chunk_large_values_and_state(flow, dt):
    """The forward passes of bf16 data round v, the running state and the
    delta-rule writes to fp16 for the MFMA (max 65504).  Values and initial
    state ~1e3 times the workloads' (|v| up to ~4e3, S0 ~ N(0, 1e3)), the
    range the header documents, still match the oracle."""
    from tests.gpu_util import run_chunk
    hk, hv, d, lens = 2, 4, 128, [150, 64, 90]
    w = gi.Workload("big", sum(lens), hk, hv, d, dt, seq="varlen", init_state=True,
                    final_state=True, seed=21)
    inp = gi.make_inputs(w, seqlens=lens, A_range=(0.01, 0.1))
    cu, T = inp["cu_seqlens"], inp["T"]
    y = _rnd(oracle.conv_fwd(inp["x"], inp["w_conv"], cu, 2 * hk * d, d), dt)
    y[:, 2 * hk * d:] = _rnd(y[:, 2 * hk * d:] * 1000.0, dt)
    g, beta = oracle.gate_fwd(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    g, beta = g.astype(np.float32), beta.astype(np.float32)
    S0 = (inp["S0"] * 1e4).astype(np.float32)          # N(0, 0.1) -> N(0, 1e3)
    rng = np.random.default_rng(22)
    dout = _rnd(rng.standard_normal((T, hv, d), dtype=np.float32), dt)
    dSf = inp["dS_T"]
    q, k, v = gi.split_qkv(y, hk, hv, d)
    scale = d ** -0.5
    o_ref, Sf_ref = oracle.delta_fwd(q, k, v, g, beta, cu, scale, S0)
    ref = oracle.delta_bwd(q, k, v, g, beta, cu, scale, dout, S0, dSf)
    assert np.max(np.abs(Sf_ref)) > 1e3 and np.max(np.abs(v)) > 2e3
    sh = L.make_shape(inp["N"], T, hk, hv, d, _gdt(dt))
    yt = dev(y, _tdt(dt))
    ws = torch.empty(L.gdn_chunk_bwd_workspace(sh), dtype=torch.uint8, device=DEV)
    r = run_chunk(flow, sh, yt[:, : hk * d], yt[:, hk * d: 2 * hk * d], yt[:, 2 * hk * d:], dev(g),
                  dev(beta), scale, dev(S0), torch.from_numpy(cu).to(DEV),
                  dev(dout, _tdt(dt)), dev(dSf), ws)
    torch.cuda.synchronize()
    got = {"o": host(r["o"]), "S_final": host(r["S_final"]),
           "dq": host(r["dq"]).reshape(T, hk, d), "dk": host(r["dk"]).reshape(T, hk, d),
           "dv": host(r["dv"]).reshape(T, hv, d), "dg": host(r["dg"]), "dbeta": host(r["dbeta"]),
           "dS0": host(r["dS0"])}
    refs = {"o": o_ref, "S_final": Sf_ref, "dq": ref[0], "dk": ref[1], "dv": ref[2], "dg": ref[3],
            "dbeta": ref[4], "dS0": ref[5]}
    errs = {k: rel_err(got[k], refs[k]) for k in refs}
    print(flow, " ".join(f"{k}={e:.2e}" for k, e in errs.items()), flush=True)
    for k in refs:
        assert_close(k, got[k], refs[k], FWD_TOL_BF16 if k in ("o", "S_final") else GRAD_TOL_BF16)


# ------------------------------------------------------------------ conv with a carried state
@pytest.mark.parametrize("name", ["fp32_ragged", "bf16_g2_mild", "bf16_d32", "fp16_d32"])
def test_conv_state_fwd_bwd(name):
    """gdn_conv_fwd_state / gdn_conv_bwd_state against the oracle, with a
    random carried state in and a random gradient of the final state; the
    final state is a copy of input rows, so it is compared exactly."""
    w, inp = _case(name)
    dt = w.dtype
    cu = inp["cu_seqlens"]
    lens = np.diff(cu)
    n_l2 = 2 * w.hk * w.d
    rng = np.random.default_rng(8)
    C = w.channels
    cs = _rnd(rng.standard_normal((len(lens), 3, C)), dt)
    dcs = _rnd(rng.standard_normal((len(lens), 3, C)), dt)
    y_ref, cs_ref = oracle.conv_state_fwd(inp["x"], inp["w_conv"], cu, n_l2, w.d, cs)
    dy = _rnd(rng.standard_normal(y_ref.shape), dt)
    dx_ref, dw_ref, dcs_ref = oracle.conv_state_bwd(inp["x"], inp["w_conv"], cu, n_l2, w.d, dy, cs,
                                                    dcs)
    sh = _shape(w, inp)
    x = dev(inp["x"], _tdt(dt))
    wc = dev(inp["w_conv"])
    cut = torch.from_numpy(cu).to(DEV)
    cst = dev(cs, _tdt(dt))
    y = torch.empty_like(x)
    cs_out = torch.empty_like(cst)
    L.gdn_conv_fwd_state(sh, x, wc, cut, y, cst, cs_out)
    dx = torch.empty_like(x)
    dw = torch.empty_like(wc)
    dcs_in = torch.empty_like(cst)
    ws = torch.empty(max(L.gdn_conv_bwd_workspace(sh), 16), dtype=torch.uint8, device=DEV)
    L.gdn_conv_bwd_state(sh, x, wc, cut, dev(dy, _tdt(dt)), dx, dw, ws, cst, dev(dcs, _tdt(dt)),
                         dcs_in)
    torch.cuda.synchronize()
    assert_close("y", host(y), y_ref, _tol(dt))
    np.testing.assert_array_equal(host(cs_out), cs_ref)
    assert_close("dx", host(dx), dx_ref, _tol(dt, True))
    assert_close("dw", host(dw), dw_ref, _tol(dt, True))
    assert_close("d_conv_state", host(dcs_in), dcs_ref, _tol(dt, True))
