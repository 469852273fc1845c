"""The seeded input generator: determinism, bf16 exactness, varlen packing."""
import numpy as np

from gated_deltanet_layer_causal_amd import inputs as gi


def test_round_bf16_is_rne_and_exact():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.3, 1e-30, 65504.0], dtype=np.float32)
    r = gi.round_bf16(x)
    # bf16 keeps 8 significant bits: low 16 bits of the float32 pattern are zero
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to even (1.0)
    assert r[1] == 1.0
    # 1 + 1.5 * 2^-8 rounds up to 1 + 2^-7
    assert r[2] == np.float32(1.0078125)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
    np.testing.assert_array_equal(gi.bits_to_f32(gi.bf16_bits(r)), r)


def test_generator_is_deterministic_and_shaped():
    w = gi.WORKLOADS["tiny"]
    a = gi.make_inputs(w)
    b = gi.make_inputs(w)
    for k in ("x", "w_conv", "a", "b", "A_log", "z", "w_norm", "dy"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["x"].shape == (64, w.channels)
    assert a["z"].shape == (64, 2, 32)
    assert np.all(np.exp(a["A_log"]) >= 1.0) and np.all(np.exp(a["A_log"]) <= 16.0)
    assert a["S0"] is None and a["dS_T"] is None


def test_varlen_lengths_cover_exactly():
    w = gi.WORKLOADS["varlen16k"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = gi.varlen_lengths(rng, 16384)
    assert sum(lens) == 16384
    assert all(512 <= L <= 4096 for L in lens[:-1]) and 1 <= lens[-1] <= 4096
    inp = gi.make_inputs(w, T=16384)
    assert inp["cu_seqlens"][0] == 0 and inp["cu_seqlens"][-1] == 16384
    assert np.all(np.diff(inp["cu_seqlens"]) > 0)


def test_bf16_workload_tensors_are_bf16_exact():
    w = gi.WORKLOADS["next4k"]
    inp = gi.make_inputs(w, T=128)
    for k in ("x", "a", "b", "z", "dy"):
        assert np.all((inp[k].view(np.uint32) & 0xFFFF) == 0), k
