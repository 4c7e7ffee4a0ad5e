"""The seeded input generator: its published definition, block addressing and
the distributions of the workloads."""
import numpy as np

import synth
from synth.workloads import WORKLOADS, gen_inputs

MASK = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def _mix64(z):
    # splitmix64 output function (Vigna), written out in Python integers
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_raw_bits_follow_splitmix64_definition():
    seed, stream = 1002, 5
    key = _mix64((seed * GOLDEN + stream) & MASK)
    ref = [_mix64((key + (i + 1) * GOLDEN) & MASK) for i in range(1000, 1010)]
    assert list(synth.raw_bits(seed, stream, 1000, 10)) == ref
    u = synth.raw_uniform(seed, stream, 1000, 10)
    np.testing.assert_array_equal(u, [(r >> 11) * 2.0 ** -53 for r in ref])


def test_splitmix64_known_sequence():
    # splitmix64 seeded with 0 yields 0xE220A8397B1DCDAF first (published test vector)
    assert _mix64(GOLDEN) == 0xE220A8397B1DCDAF


def test_blocks_equal_slices_of_full_tensor():
    wl = WORKLOADS["k3_layer"]
    full = gen_inputs(wl, time=(100, 40), heads=(40, 16))
    part = gen_inputs(wl, time=(110, 20), heads=(45, 6))
    for key in ("q", "k", "v", "z", "gate"):
        assert np.array_equal(full[key][:, 10:30, 5:11], part[key]), key
    assert np.array_equal(full["beta"][:, 10:30, 5:11], part["beta"])
    # the pinned half of the heads of this workload
    z = synth.bf16_bits_to_f32(full["z"])
    assert np.all(z[:, :, 48 - 40:] == 30.0) and np.all(np.abs(z[:, :, : 48 - 40]) < 8)


def test_distributions():
    wl = WORKLOADS["prefill"]
    x = gen_inputs(wl, batch=(1, 1), time=(0, 512))
    q = synth.bf16_bits_to_f32(x["q"]).astype(np.float64)
    nrm = np.linalg.norm(q, axis=-1)
    assert np.all(np.abs(nrm - 1) < 0.01)
    v = synth.bf16_bits_to_f32(x["v"]).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    z = synth.bf16_bits_to_f32(x["z"]).astype(np.float64)
    assert abs(z.std() - 2) < 0.02
    b = synth.bf16_bits_to_f32(x["beta"]).astype(np.float64)
    assert b.min() > 0 and b.max() < 1 and abs(b.mean() - 0.5) < 0.01
    assert np.all(np.abs(x["A"]) <= 1) and x["A"].std() > 0.3
    d = gen_inputs(WORKLOADS["decode"], batch=(0, 2), time=(0, 1), heads=(0, 4))
    assert d["S0"].dtype == np.float32 and abs(d["S0"].std() - 0.1) < 0.005


def test_seeds_differ_and_repeat():
    a = gen_inputs(WORKLOADS["tiny"])
    b = gen_inputs(WORKLOADS["tiny"])
    c = gen_inputs(WORKLOADS["prefill"], batch=(0, 1), time=(0, 128), heads=(0, 2))
    assert np.array_equal(a["v"], b["v"])
    assert not np.array_equal(a["v"][..., :64], synth.bf16_bits_to_f32(c["v"])[..., :64])


def test_bf16_rounding_helper():
    x = np.array([1.0, 1.00390625, 1.01171875, -3.3e38, 1e-40], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0  # tie rounds to even
    assert back[2] == np.float32(1.015625)
