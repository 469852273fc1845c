"""Seeded synthetic inputs for the Gated DeltaNet layer core.

This module is shared by the tests, the bench and the oracle's callers.  It
holds none of the method's arithmetic: it only draws random tensors with the
shapes and distributions of the workloads, rounds them to bfloat16 where the
workload is bf16, and packs ``cu_seqlens``.

Workloads (Gated DeltaNet core, head dim 128 unless stated):

* ``tiny``      T=64, one sequence, 1 k-head / 2 v-heads, d=32, fp32.
* ``next4k``    T=4096, one sequence, 16 k-heads / 32 v-heads, bf16
                (Qwen3-Next-shaped, the Megatron page's GDN arguments).
* ``varlen16k`` 16384 tokens packed from sequences of length U{512..4096},
                the last truncated to fit; 16 k-heads / 48 v-heads, bf16
                (Qwen3.8-Flash-shaped heads from the miles page).
* ``tp4share``  T=65536, one sequence, 4 k-heads / 8 v-heads, bf16, nonzero
                initial state N(0, 0.1) and the final state returned (one
                GPU's head share of a 16/32 model at four-way head sharding).
* ``long128k``  T=131072, one sequence, 16 k-heads / 48 v-heads, bf16.
* ``flash64k``  T=65536, one sequence, 16 k-heads / 48 v-heads, bf16: the
                Qwen3.8-Flash GDN shape at 64k tokens used for throughput.

Distributions: pre-conv q, k, v ~ N(0, 1); conv weights ~ N(0, 0.25)
(0.25 read as the standard deviation); gate input a ~ N(0, 1) with
A ~ U(1, 16), A_log = log A, dt_bias = 0; beta input b ~ N(0, 1); output
gate z ~ N(0, 1); norm weight ~ N(0, 0.1); upstream gradients ~ N(0, 1).
Draw order (one numpy PCG64 stream): sequence lengths (varlen only), x,
w_conv, a, b, A, z, w_norm, S0, dy, dS_T.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CONV_K = 4
CHUNK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hk: int
    hv: int
    d: int
    dtype: str               # "bf16", "fp16" or "fp32": storage type of token tensors
    seq: str = "single"      # "single" or "varlen"
    init_state: bool = False  # nonzero S0 ~ N(0, 0.1)
    final_state: bool = False  # S_final returned, upstream grad dS_T ~ N(0, 1)
    seed: int = 1000
    A_range: tuple = (1.0, 16.0)   # A ~ U(lo, hi); A_log = log A

    @property
    def channels(self) -> int:
        return 2 * self.hk * self.d + self.hv * self.d


WORKLOADS = {
    "tiny": Workload("tiny", 64, 1, 2, 32, "fp32", seed=1000),
    "next4k": Workload("next4k", 4096, 16, 32, 128, "bf16", seed=1001),
    "varlen16k": Workload("varlen16k", 16384, 16, 48, 128, "bf16", seq="varlen", seed=1002),
    "tp4share": Workload("tp4share", 65536, 4, 8, 128, "bf16", init_state=True,
                         final_state=True, seed=1003),
    "long128k": Workload("long128k", 131072, 16, 48, 128, "bf16", seed=1004),
    "flash64k": Workload("flash64k", 65536, 16, 48, 128, "bf16", seed=1005),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def round_fp16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest float16 (ties to even); returns
    float32 values exactly representable in float16 (|x| > 65504 -> inf)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to(dtype: str):
    """The rounding of token tensors stored as `dtype` ("bf16", "fp16",
    "fp32"), or None for fp32."""
    return {"bf16": round_bf16, "fp16": round_fp16, "fp32": None}[dtype]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The uint16 bfloat16 bit patterns of bf16-exact float32 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def varlen_lengths(rng: np.random.Generator, total: int, lo: int = 512, hi: int = 4096) -> list:
    """Integer lengths ~ U{lo..hi} drawn until they cover ``total``; the last
    one is truncated so that the lengths sum to exactly ``total``."""
    lens = []
    s = 0
    while s < total:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, total - s)
        lens.append(L)
        s += L
    return lens


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64)).astype(np.int32)
    return cu


def make_inputs(w: Workload, T: Optional[int] = None, seqlens=None, seed: Optional[int] = None,
                A_range: Optional[tuple] = None, dtype: Optional[str] = None) -> dict:
    """Draw one set of layer inputs for workload ``w``.

    ``T`` / ``seqlens`` override the token count (for scaled-down parity
    cases); ``A_range`` overrides the gate's A distribution (mild decay keeps
    state alive across many chunks).  All token tensors are float32 arrays;
    for bf16 / fp16 workloads they are exact in that type.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    dt = w.dtype if dtype is None else dtype
    if seqlens is not None:
        lens = list(seqlens)
        T = int(sum(lens))
    elif w.seq == "varlen":
        T = w.T if T is None else T
        lens = varlen_lengths(rng, T)
    else:
        T = w.T if T is None else T
        lens = [T]
    cu = cu_from_lengths(lens)
    N = len(lens)
    C = w.channels
    Hv, d = w.hv, w.d
    lo, hi = w.A_range if A_range is None else A_range

    def f32(shape, std=1.0):
        a = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return a

    out = {"cu_seqlens": cu, "T": T, "N": N}
    out["x"] = f32((T, C))
    out["w_conv"] = f32((C, CONV_K), 0.25)
    out["a"] = f32((T, Hv))
    out["b"] = f32((T, Hv))
    A = rng.uniform(lo, hi, size=Hv).astype(np.float64)
    out["A_log"] = np.log(A).astype(np.float32)
    out["dt_bias"] = np.zeros(Hv, dtype=np.float32)
    out["z"] = f32((T, Hv, d))
    out["w_norm"] = f32((d,), 0.1)
    out["S0"] = f32((N, Hv, d, d), 0.1) if w.init_state else None
    out["dy"] = f32((T, Hv, d))
    out["dS_T"] = f32((N, Hv, d, d)) if w.final_state else None
    rnd = round_to(dt)
    if rnd is not None:
        for key in ("x", "a", "b", "z", "dy"):
            out[key] = rnd(out[key])
    out["dtype"] = dt
    return out


def split_qkv(y: np.ndarray, hk: int, hv: int, d: int):
    """Views of q [T,Hk,d], k [T,Hk,d], v [T,Hv,d] inside a [T, C] tensor laid
    out q | k | v, head-major inside each block."""
    T = y.shape[0]
    q = y[:, : hk * d].reshape(T, hk, d)
    k = y[:, hk * d: 2 * hk * d].reshape(T, hk, d)
    v = y[:, 2 * hk * d:].reshape(T, hv, d)
    return q, k, v
