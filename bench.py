"""Throughput of the Gated DeltaNet layer core (forward + backward) on one GPU.

One step = conv -> gate -> chunked gated delta rule -> gated norm forward,
then the four backward calls, over one batch of synthetic input already
resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload flash64k]

Per-call durations are measured with HIP events recorded on the stream the
calls are launched on (torch's current stream) across the timed steps; the
dominant call is reported against its roofline with the algorithmic work
per token of that call (bytes for HBM-bound calls, flops for MFMA-bound ones).
The CPU oracle is timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN fwd+bwd tokens/s (16k/48v heads, d=128, 64k tok); % MFMA/HBM peak"
FORWARD_CALLS = ("conv_fwd", "gate_fwd", "chunk_prepare", "chunk_fwd_states", "norm_fwd")
# calls that launch more than one kernel (not used for the single-kernel roofline)
MULTI_KERNEL_CALLS = ("chunk_fwd_states", "chunk_prepare", "chunk_prepare_b", "chunk_bwd_states",
                      "conv_bwd", "norm_bwd", "gate_bwd")
# HIP sources of the kernel behind each single-kernel call (HBM traffic taken
# from committed counter summaries is used only while these are unchanged)
KERNEL_SOURCES = {
    "chunk_bwd_grads": ["chunk_grad.hip", "chunk_stream.h", "chunk_common.h", "common.h", "launch.h"],
    "chunk_bwd_reverse": ["chunk_rev.hip", "chunk_stream.h", "chunk_common.h", "common.h",
                          "launch.h"],
    "conv_fwd": ["conv.hip", "common.h", "launch.h"],
    "norm_fwd": ["norm.hip", "common.h", "launch.h"],
    "gate_fwd": ["gate.hip", "common.h", "launch.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_flash64k.txt")


def sources_digest(call):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(call, []):
        with open(os.path.join(ROOT, "gated_deltanet_layer_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(call):
    """HBM bytes per launch of `call` from the committed counter summary, or
    None when there is none or the kernel's sources changed since."""
    if call not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    for line in open(TRAFFIC_FILE):
        if not line.startswith("call="):
            continue
        kv = dict(f.split("=", 1) for f in line.split())
        if kv.get("call") == call and kv.get("sources") == sources_digest(call):
            return float(kv["hbm_bytes_per_launch"])
    return None
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3

# Algorithmic work per token of each call (E = bytes per element of the
# token tensors).  HBM-bound calls count the bytes they must read and write.
# The chunk phases count the dense contraction flops of the products they
# form (chunk C = 64, head dim d, per value head unless noted):
#   fwd_states : W S^T, Q S^T, S update (3 x 2 d^2) + M V, P Delta (2 x 2 C d)
#   fwd_states_save: the saved-state pass, K S^T and the S update (2 x 2 d^2)
#                + M R (2 C d), which also stores R and Delta for 16-bit data,
#                then the outputs: Q S^T (2 d^2) + P Delta (2 C d) (fp32 data:
#                K S^T, Q S^T (2 x 2 d^2) + M R, P Delta (2 x 2 C d))
#   bwd_states : the saved-state pass (fp32 data: + K S^T, M R)
#   bwd_reverse: K dS'^T, Q^T dO, K^T dR (3 x 2 d^2) + P^T dO, M^T dDelta (2 x 2 C d)
#   bwd_grads  : dO S, dR S, Delta dS' (3 x 2 d^2); dM, dP in both
#                orientations, (dP o D) K, (dP o D)^T Q and WS K, WS = WA + WA^T
#                forming (dA o bD) K + (dA o bD)^T K in one product
#                (6 x 2 C d); Tinv products (2 x 2 C^2); K K^T comes from the
#                preparation
# The preparation is bandwidth-bound; its algorithmic bytes are its inputs
# q, k, g, beta (its writes are intermediates).
def algorithmic_per_token(name, hk, hv, d, E, saved=True):
    C = 2 * hk * d + hv * d
    C64 = 64
    if name == "conv_fwd":
        return "hbm", 2 * C * E                       # read x, write y
    if name == "conv_bwd":
        return "hbm", 3 * C * E                       # read x, dy; write dx
    if name == "gate_fwd":
        return "hbm", hv * (2 * E + 8)                # read a, b; write g, beta
    if name == "gate_bwd":
        return "hbm", hv * (2 * E + 8 + 2 * E)        # read a, b, dg, dbeta; write da, db
    if name == "norm_fwd":
        return "hbm", 3 * hv * d * E                  # read o, z; write y
    if name == "norm_bwd":
        return "hbm", 5 * hv * d * E                  # read o, z, dy; write do, dz
    # preparation: reads q, k (per key head) and g, beta (per value head); per
    # value head writes gamma (fp64), Gam and dec (fp32), M and P.  Forward
    # mode adds, per key head, K^T and the Q rows in the compute type and, per
    # value head, W.  Backward mode adds per key head the K rows, K^T and Q^T
    # in the storage type and one more key-head tile (the K rows in the
    # compute type for 16-bit data, the compute-type K^T for fp32), per value
    # head P^T, Tinv, Tinv^T and beta (and W for fp32).
    # The method needs only q, k, g and beta from memory here: everything the
    # preparation writes is an intermediate of this implementation, so it
    # counts none of it (its traffic is reported beside, from the counters).
    if name in ("chunk_prepare", "chunk_prepare_b"):
        return "hbm", 2 * hk * d * E + 2 * hv * 4
    # products formed per v-head token: the forward pass without saved
    # states (W S^T, Q S^T, update; M V, P Delta); the saved-state pass (K S^T,
    # update; M R for 16-bit data, W S^T, update; M V for fp32) and the
    # chunk-parallel outputs: for 16-bit data Q S^T and P Delta (the pass has
    # stored R and Delta), for fp32 K S^T, Q S^T; M R, P Delta, whose O part
    # the recompute flow leaves out
    fwd_states = hv * (6 * d * d + 4 * C64 * d)
    save_pass = hv * (4 * d * d + 2 * C64 * d)
    if E == 2:   # the saved-state pass stores R and Delta: O alone remains
        outputs = hv * (2 * d * d + 2 * C64 * d)
        outputs_no_o = 0
    else:
        outputs = hv * (4 * d * d + 4 * C64 * d)
        outputs_no_o = hv * (2 * d * d + 2 * C64 * d)
    if name == "chunk_fwd_states":
        return "mfma", (save_pass + outputs) if saved else fwd_states
    if name == "chunk_bwd_states":
        return "mfma", save_pass + outputs_no_o
    if name == "chunk_bwd_reverse":
        return "mfma", hv * (6 * d * d + 4 * C64 * d)
    if name == "chunk_bwd_grads":
        return "mfma", hv * (6 * d * d + 12 * C64 * d + 4 * C64 * C64)
    raise KeyError(name)


# Floors of the layer at 100% of peak (the scope table's per-token counts):
#   chunked rule, per value head and token: forward 10 C d + 6 d^2 + 2/3 C^2,
#     backward 30 C d + 16 d^2 flop (dense tiles, C = 64); bytes: q, k, v, g,
#     beta in and o out (forward), q, k, v, g, beta, do in and dq, dk, dv, dg,
#     dbeta out (backward);
#   conv fwd+bwd 5 C_ch E, gate hv (6 E + 16), norm 8 hv d E + 4 hv bytes.
def layer_floor(hk, hv, d, E, T, peak_tflops):
    C64 = 64
    chunk_flop = hv * (10 * C64 * d + 6 * d * d + 2 * C64 * C64 / 3 + 30 * C64 * d + 16 * d * d)
    chunk_bytes = (2 * hk * d * E + 2 * hv * d * E + 8 * hv) + \
                  (2 * hk * d * E + 2 * hv * d * E + 8 * hv + 2 * hk * d * E + hv * d * E + 8 * hv)
    Cch = 2 * hk * d + hv * d
    hbm_bytes = 5 * Cch * E + hv * (6 * E + 16) + 8 * hv * d * E + 4 * hv
    chunk_ms = max(chunk_flop * T / (peak_tflops * 1e12), chunk_bytes * T / (HBM_PEAK_GBS * 1e9)) * 1e3
    other_ms = hbm_bytes * T / (HBM_PEAK_GBS * 1e9) * 1e3
    return {"chunk_ms": chunk_ms, "conv_gate_norm_ms": other_ms, "layer_ms": chunk_ms + other_ms,
            "chunk_mflop_per_token": chunk_flop / 1e6, "chunk_bytes_per_token": chunk_bytes}


# Counter summaries of the chunk kernels (MFMA busy fraction and executed
# MFMA flops per launch, from rocprofv3 --pmc), used while the kernel's
# sources are unchanged since they were taken.
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_flash64k.txt")
KERNEL_FILES = {
    "chunk_grad": ["chunk_grad.hip"], "chunk_rev": ["chunk_rev.hip"],
    "chunk_state[m1]": ["chunk_state.hip"], "chunk_o": ["chunk_out.hip"],
    "chunk_prep[bwd]": ["chunk_fwd.hip"],
}
CALL_KERNELS = {"chunk_bwd_grads": ["chunk_grad"], "chunk_bwd_reverse": ["chunk_rev"],
                "chunk_fwd_states": ["chunk_state[m1]", "chunk_o"],
                "chunk_prepare": ["chunk_prep[bwd]"]}


def kernel_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_FILES[kernel] + ["chunk_stream.h", "chunk_common.h", "common.h", "launch.h"]:
        with open(os.path.join(ROOT, "gated_deltanet_layer_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mfma_counters():
    """kernel -> {"mfma_util": %, "exec_flop": flop per launch} from the
    committed summary, for kernels whose sources still match."""
    out = {}
    if not os.path.exists(MFMA_FILE):
        return out
    for line in open(MFMA_FILE):
        if not line.startswith("kernel="):
            continue
        kv = dict(f.split("=", 1) for f in line.split())
        kname = kv["kernel"]
        if kname in KERNEL_FILES and kv.get("sources") == kernel_digest(kname):
            out[kname] = {"mfma_util": float(kv["mfma_util"]), "exec_flop": float(kv["exec_flop"])}
    return out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="flash64k")
    p.add_argument("--seed", type=int, default=1005)
    p.add_argument("--cpu-sample-tokens", type=int, default=16384)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--seg-chunks", type=int, default=0,
                   help="segment length (chunks) of the segment-parallel state scan: 0 lets the "
                        "library decide, < 0 keeps one sequential pass per sequence")
    p.add_argument("--proj-hidden", type=int, default=None,
                   help="hidden size of the layer with its in/out projections, timed beside the "
                        "core (0: skip; default: 2560 for the 16 k / 48 v-head shapes, the "
                        "Qwen3.8-Flash layer, else skip)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain bf16 device copy of MIB MiB three times (reference "
                        "for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 2, "bytes_written": n * 2,
                                           "kib": n * 2 / 1024, "launches": 3}}), flush=True)


def make_gpu_inputs(w, seed, dev):
    """Synthetic inputs with the workload's distributions, drawn on the GPU
    from a seeded generator (same distributions as the numpy generator)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    bf = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, C, Hv, d = w.T, w.channels, w.hv, w.d

    def n(shape, std=1.0, dt=torch.float32):
        return (torch.randn(shape, generator=g, device=dev) * std).to(dt)

    A = torch.rand(Hv, generator=g, device=dev) * (w.A_range[1] - w.A_range[0]) + w.A_range[0]
    inp = {
        "x": n((T, C), dt=bf), "w_conv": n((C, 4), 0.25), "a": n((T, Hv), dt=bf),
        "b": n((T, Hv), dt=bf), "A_log": torch.log(A), "dt_bias": torch.zeros(Hv, device=dev),
        "z": n((T, Hv, d), dt=bf), "w_norm": n((d,), 0.1), "dy": n((T, Hv, d), dt=bf),
        "cu_seqlens": torch.tensor([0, T], dtype=torch.int32, device=dev),
    }
    if w.seq == "varlen":
        # the packed lengths are drawn as the parity tests draw them
        import numpy as np
        from gated_deltanet_layer_causal_amd import inputs as gi
        lens = gi.varlen_lengths(np.random.Generator(np.random.PCG64(w.seed)), T)
        inp["cu_seqlens"] = torch.from_numpy(gi.cu_from_lengths(lens)).to(dev)
    if w.init_state:
        inp["S0"] = n((1, Hv, d, d), 0.1)
    if w.final_state:
        inp["dS_T"] = n((1, Hv, d, d))
    return inp


class EventTimer:
    """Records a HIP event before and after each named call on the current stream."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pairs = {}
        self.active = False

    def __call__(self, name, phase):
        if not self.active:
            return
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(self.torch.cuda.current_stream())
        self.pairs.setdefault(name, []).append(ev)  # begin, end, begin, end, ...

    def mean_ms(self):
        out = {}
        for name, evs in self.pairs.items():
            ts = [evs[i].elapsed_time(evs[i + 1]) for i in range(0, len(evs) - 1, 2)]
            out[name] = sum(ts) / len(ts)
        return out


# Per-layer forward+backward of Qwen3.8-Flash's GDN layer (hidden 2560, 16 k /
# 48 v heads) at TP=1 on one H200, 64k tokens, as printed on the miles page
# (H200 results): another machine's figure, with the projections; context only.
PAGES_H200_LAYER_MS_64K = 52.6


def layer_with_projections(w, hidden, inp, steps, warmup, dev):
    """The layer with its in/out projections (library GEMMs around the core),
    forward+backward, timed like the core.  Returns the JSON object."""
    import torch
    from gated_deltanet_layer_causal_amd.layer import CoreConfig, GDNLayer
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    bf = torch.bfloat16
    T, C, Hv, d = w.T, w.channels, w.hv, w.d
    shapes = {"x": (C, hidden), "z": (Hv * d, hidden), "a": (Hv, hidden), "b": (Hv, hidden),
              "out": (hidden, Hv * d)}
    W = {k: (torch.randn(s, generator=g, device=dev) / math.sqrt(s[1])).to(bf) for k, s in shapes.items()}
    layer = GDNLayer(CoreConfig(hk=w.hk, hv=w.hv, d=w.d, dtype=bf), hidden, W, device=dev)
    X = torch.randn((T, hidden), generator=g, device=dev).to(bf)
    dY = torch.randn((T, hidden), generator=g, device=dev).to(bf)
    pa = (inp["w_conv"], inp["A_log"], inp["dt_bias"], inp["w_norm"], inp["cu_seqlens"])
    timer = EventTimer()

    def step():
        f = layer.forward(X, *pa, timer=timer)
        layer.backward(f, X, *pa, dY, timer=timer)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.active = True
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    pc = timer.mean_ms()
    gemm_ms = sum(pc[k] for k in ("in_proj", "out_proj", "in_proj_bwd", "out_proj_bwd"))
    n_out = C + Hv * d + 2 * Hv
    gemm_flop = 3 * 2 * T * hidden * (n_out + Hv * d)    # forward, input and weight gradients
    return {"hidden": hidden, "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms / 1e3), 1),
            "gemm_ms": round(gemm_ms, 4), "gemm_tflops": round(gemm_flop / (gemm_ms / 1e3) / 1e12, 1),
            "gemm_frac_bf16_peak": round(gemm_flop / (gemm_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "gemms": "torch.matmul (hipBLASLt), bf16, fp32 accumulate",
            "pages_h200_ms_per_layer": PAGES_H200_LAYER_MS_64K if T == 65536 else None,
            "note": "in_proj -> core -> out_proj, forward and backward with all weight gradients; "
                    "the pages' figure is another machine's (context, not a target)"}


def cpu_baseline(w, sample_T, core, dev):
    """The oracle's layer forward+backward on the first sample_T tokens of the
    workload (timed), and the GPU core on the same inputs (outside every
    timed region) compared with it: per-tensor max relative error,
    max|gpu - oracle| / max|oracle|."""
    import numpy as np
    import torch
    import oracle
    from gated_deltanet_layer_causal_amd import inputs as gi
    inp = gi.make_inputs(w, T=sample_T)
    rf = gi.round_to(w.dtype)
    t0 = time.perf_counter()
    f = oracle.layer_fwd(inp, w.hk, w.hv, w.d, w.d ** -0.5, round_fn=rf)
    b = oracle.layer_bwd(inp, f, w.hk, w.hv, w.d, w.d ** -0.5, round_fn=rf)
    dt = time.perf_counter() - t0
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]

    def t(a, dtype=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(dtype)

    args = (t(inp["x"], tdt), t(inp["w_conv"]), t(inp["a"], tdt), t(inp["b"], tdt),
            t(inp["A_log"]), t(inp["dt_bias"]), t(inp["z"], tdt), t(inp["w_norm"]),
            torch.from_numpy(inp["cu_seqlens"]).to(dev))
    S0 = t(inp["S0"]) if inp["S0"] is not None else None
    dST = t(inp["dS_T"]) if inp["dS_T"] is not None else None
    gf = core.forward(*args, S0=S0, want_final=True)
    gb = core.backward(gf, *args, t(inp["dy"], tdt), S0=S0, dS_final=dST)
    torch.cuda.synchronize()
    errs = {}
    for key, got, ref in [(k, gf[k], f[k]) for k in ("y", "o", "out", "S_final")] + \
                         [(k, gb[k], b[k]) for k in ("dy_conv", "dx", "dw_conv", "dz", "da", "db",
                                                     "dA_log", "ddt_bias", "dw_norm", "dS0")]:
        g_ = got.detach().float().cpu().numpy().astype(np.float64).reshape(np.shape(ref))
        errs[key] = float(np.max(np.abs(g_ - ref)) / max(np.max(np.abs(ref)), 1e-300))
    return {"value": sample_T / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"layer fwd+bwd on the first {sample_T} tokens of the {w.name} shape "
                      f"({w.hk}k/{w.hv}v heads, d={w.d}), fp64 token-by-token, {dt:.1f} s",
            "max_rel_err_gpu_vs_oracle": {k: float(f"{v:.3e}") for k, v in errs.items()}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer core "
              "is head-parallel: a multi-GPU run would give each GPU a group of key heads with "
              "their value heads, with no exchange inside the core)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    from gated_deltanet_layer_causal_amd import inputs as gi
    from gated_deltanet_layer_causal_amd.layer import CoreConfig, GDNCore

    w = gi.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    core = GDNCore(CoreConfig(hk=w.hk, hv=w.hv, d=w.d, dtype=dt, seg_chunks=args.seg_chunks),
                   device=dev)
    inp = make_gpu_inputs(w, args.seed, dev)
    args_f = (inp["x"], inp["w_conv"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"], inp["z"],
              inp["w_norm"], inp["cu_seqlens"])
    timer = EventTimer()

    def step():
        f = core.forward(*args_f, S0=inp.get("S0"), want_final=w.final_state, timer=timer)
        core.backward(f, *args_f, inp["dy"], S0=inp.get("S0"), dS_final=inp.get("dS_T"),
                      timer=timer)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` steps between two events, with an
    # event at every step boundary for the median
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    timer.active = True
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    timer.active = False
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    value = w.T / (ms / 1e3)
    per_call = timer.mean_ms()
    # the same steps with the 256 MB last-level cache flushed before each
    # (a 512 MB write between steps), timed per step only
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flushed = []
    for _ in range(args.steps):
        flush.zero_()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        step()
        b_.record()
        flushed.append((a_, b_))
    torch.cuda.synchronize()
    flushed_ms = sorted(a_.elapsed_time(b_) for a_, b_ in flushed)
    del flush

    E = 4 if w.dtype == "fp32" else 2
    single = {k: v for k, v in per_call.items() if k not in MULTI_KERNEL_CALLS}
    dom = max(single, key=single.get)
    bound, per_tok = algorithmic_per_token(dom, w.hk, w.hv, w.d, E)
    if bound == "hbm":
        achieved = per_tok * w.T / (per_call[dom] / 1e3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = per_tok * w.T / (per_call[dom] / 1e3) / 1e12
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        unit = "TFLOP/s"
    fwd_ms = sum(t for k, t in per_call.items() if k in FORWARD_CALLS)
    bwd_ms = sum(t for k, t in per_call.items() if k not in FORWARD_CALLS)
    calls = {}
    counters = mfma_counters() if (w.name, w.dtype) == ("flash64k", "bf16") else {}
    for name, t in sorted(per_call.items(), key=lambda kv: -kv[1]):
        b, pt = algorithmic_per_token(name, w.hk, w.hv, w.d, E)
        rate = pt * w.T / (t / 1e3) / (1e9 if b == "hbm" else 1e12)
        pk = HBM_PEAK_GBS if b == "hbm" else (BF16_PEAK_TFLOPS if E == 2 else FP32_PEAK_TFLOPS)
        calls[name] = {"ms": round(t, 4), "bound": b, "achieved": round(rate, 2),
                       "frac": round(rate / pk, 4)}
        # counter figures of the call's kernels (MFMA busy %, executed MFMA
        # flops per launch), where the committed summary matches the sources
        ks = [k for k in CALL_KERNELS.get(name, []) if k in counters]
        if ks:
            calls[name]["counters"] = {k: counters[k] for k in ks}
    peak_mm = BF16_PEAK_TFLOPS if E == 2 else FP32_PEAK_TFLOPS
    floor = layer_floor(w.hk, w.hv, w.d, E, w.T, peak_mm)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded on-device draws with the workload's distributions)",
        "config": {"workload": f"{w.name}: GDN layer core fwd+bwd, {w.hk} k-heads / {w.hv} v-heads, "
                               f"d={w.d}, {w.T} tokens, "
                               f"{'varlen pack' if w.seq == 'varlen' else 'single sequence'}, chunk 64",
                   "tokens": w.T, "hk": w.hk, "hv": w.hv, "d": w.d, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom),
                     "kernel": dom, "ms_per_launch": round(per_call[dom], 4)},
        "median_ms_per_step": round(step_ms[len(step_ms) // 2], 4),
        "median_ms_per_step_llc_flushed": round(flushed_ms[len(flushed_ms) // 2], 4),
        "floor": {"layer_ms": round(floor["layer_ms"], 4), "chunk_ms": round(floor["chunk_ms"], 4),
                  "conv_gate_norm_ms": round(floor["conv_gate_norm_ms"], 4),
                  "frac": round(floor["layer_ms"] / ms, 4),
                  "note": "layer floor at 100% of MFMA/HBM peak from the algorithmic per-token "
                          "counts, over the measured step"},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "peak_mem_gib": round(torch.cuda.max_memory_allocated() / 2**30, 2),
        "calls": calls,
    }
    hidden = args.proj_hidden
    if hidden is None:
        hidden = 2560 if (w.hk, w.hv, w.d) == (16, 48, 128) else 0
    if hidden > 0 and w.dtype == "bf16":
        out["layer_with_projections"] = layer_with_projections(w, hidden, inp, args.steps,
                                                               args.warmup, dev)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens, core, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
