"""gdn_conv_bwd_noalloc (the conv backward with the library's own scratch,
for callers that cannot allocate) against gdn_conv_bwd with a caller
workspace, through the C ABI: two calls in a row, the second on a smaller
input, each bitwise equal to the workspace entry point (same kernels, same
fixed reduction order).  A third call repeats the first shape, so the
scratch the second call left behind is reused."""
import numpy as np
import pytest
import torch

from gated_deltanet_layer_causal_amd import capi as L
from gated_deltanet_layer_causal_amd import inputs as gi
from tests.gpu_util import DEV, dev

pytestmark = pytest.mark.gpu


def _case(hk, hv, d, dt, lens, seed):
    w = gi.Workload("na", sum(lens), hk, hv, d, dt, seq="varlen", seed=seed)
    inp = gi.make_inputs(w, seqlens=lens)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    T = inp["T"]
    sh = L.make_shape(inp["N"], T, hk, hv, d, L.GDN_BF16 if dt == "bf16" else L.GDN_FP32)
    x = dev(inp["x"], tdt)
    wc = dev(inp["w_conv"])
    cu = torch.from_numpy(inp["cu_seqlens"]).to(DEV)
    rng = np.random.default_rng(seed + 1)
    dy = dev(rng.standard_normal(inp["x"].shape).astype(np.float32), tdt)
    return sh, x, wc, cu, dy


def _both(sh, x, wc, cu, dy):
    ws = torch.empty(max(L.gdn_conv_bwd_workspace(sh), 16), dtype=torch.uint8, device=DEV)
    dx_ref, dw_ref = torch.empty_like(x), torch.empty_like(wc)
    L.gdn_conv_bwd(sh, x, wc, cu, dy, dx_ref, dw_ref, ws)
    dx, dw = torch.full_like(x, float("nan")), torch.full_like(wc, float("nan"))
    L.gdn_conv_bwd_noalloc(sh, x, wc, cu, dy, dx, dw)
    torch.cuda.synchronize()
    return (dx, dw), (dx_ref, dw_ref)


def test_conv_bwd_noalloc_matches_workspace_entry_point():
    cases = [
        # a large call (16 k / 48 v heads, a varlen pack of 16384 tokens), then a small one
        (16, 48, 128, "bf16", gi.varlen_lengths(np.random.Generator(np.random.PCG64(1002)), 16384), 3),
        (2, 6, 128, "bf16", [300, 65, 7, 1, 130], 4),
        (16, 48, 128, "bf16", gi.varlen_lengths(np.random.Generator(np.random.PCG64(1002)), 16384), 3),
        (1, 2, 32, "fp32", [100, 37, 1, 70], 5),
    ]
    for i, (hk, hv, d, dt, lens, seed) in enumerate(cases):
        sh, x, wc, cu, dy = _case(hk, hv, d, dt, lens, seed)
        need = L.gdn_conv_bwd_workspace(sh)
        assert need <= L.CONV_BWD_NOALLOC_MAX_BYTES
        print(f"[no-alloc call {i}] {sum(lens)} tokens, {hk}/{hv} heads, d={d}, {dt}, "
              f"scratch {need} bytes", flush=True)
        (dx, dw), (dx_ref, dw_ref) = _both(sh, x, wc, cu, dy)
        assert torch.equal(dx.view(torch.uint8), dx_ref.view(torch.uint8)), f"call {i}: dx differs"
        assert torch.equal(dw.view(torch.uint8), dw_ref.view(torch.uint8)), f"call {i}: dw differs"


def test_conv_bwd_noalloc_refuses_too_large_shapes():
    sh = L.make_shape(1, 262144, 16, 48, 128, L.GDN_BF16)
    assert L.gdn_conv_bwd_workspace(sh) > L.CONV_BWD_NOALLOC_MAX_BYTES
    C = 2 * 16 * 128 + 48 * 128
    x = torch.empty((262144, C), dtype=torch.bfloat16, device=DEV)
    wc = torch.zeros((C, 4), dtype=torch.float32, device=DEV)
    cu = torch.tensor([0, 262144], dtype=torch.int32, device=DEV)
    dw = torch.empty_like(wc)
    with pytest.raises(L.GDNError) as ei:
        L.gdn_conv_bwd_noalloc(sh, x, wc, cu, x, x, dw)
    assert ei.value.status == 4
