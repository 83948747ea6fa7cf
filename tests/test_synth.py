"""The seeded generators against an independent pure-Python restatement of
their definition (SplitMix64 counters, Box-Muller, bf16 round-to-nearest-even)."""
import math
import struct

import numpy as np
import torch

import synth

MASK = (1 << 64) - 1


def py_mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def py_at(key, i):
    return py_mix((key + (i + 1) * 0x9E3779B97F4A7C15) & MASK)


def py_normal_f32(seed, stream, i, std=0.02):
    key = py_at(seed, stream)
    u1 = (py_at(key, 2 * i) >> 11) * 2.0 ** -53
    u2 = (py_at(key, 2 * i + 1) >> 11) * 2.0 ** -53
    z = math.sqrt(-2.0 * math.log(1.0 - u1)) * math.cos(2.0 * math.pi * u2)
    return struct.unpack("f", struct.pack("f", std * z))[0]


def test_splitmix_counter_matches_definition():
    for key in (0, 1, 0x5EED0001, MASK):
        for i in (0, 1, 2, 1000, 1 << 40):
            assert synth.at(key, i) == py_at(key, i)
    assert synth.key(7, 9) == py_at(7, 9)


def test_splitmix_stream_is_the_sequential_generator():
    # A SplitMix64 generator seeded with s: state += gamma; output mix(state).
    state, key = 12345, 12345
    for i in range(10):
        state = (state + 0x9E3779B97F4A7C15) & MASK
        assert synth.at(key, i) == py_mix(state)


def test_normal_values_match_definition():
    seed, stream = synth.SEED_WEIGHTS, synth.stream_weight(synth.T_WQ, 3)
    got = synth.normal_f32(seed, stream, 64, first=100)
    want = np.array([py_normal_f32(seed, stream, 100 + i) for i in range(64)], dtype=np.float32)
    np.testing.assert_array_equal(got, want)


def test_bf16_stream_is_rne_of_f32_stream():
    seed, stream = 99, 5
    f = synth.normal_f32(seed, stream, 4096)
    b = synth.normal_bf16_bits(seed, stream, 4096)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_normal_moments():
    x = synth.normal_f32(3, 4, 1 << 20).astype(np.float64)
    assert abs(x.mean()) < 4 * 0.02 / 1024
    assert abs(x.std() - 0.02) < 0.02 * 0.005
    # fourth moment of a normal is 3 sigma^4
    k = np.mean((x / x.std()) ** 4)
    assert abs(k - 3.0) < 0.05


def test_tokens_and_uniforms():
    t = synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(0), 32000, 10000)
    assert t.min() >= 0 and t.max() < 32000
    key = py_at(synth.SEED_PROMPTS, synth.stream_prompt(0))
    assert [int(v) for v in t[:8]] == [py_at(key, i) % 32000 for i in range(8)]
    u = synth.uniforms(synth.SEED_UNIFORMS, synth.stream_uniform(2, 7), 1000)
    assert (u >= 0).all() and (u < 1).all()
    key = py_at(synth.SEED_UNIFORMS, synth.stream_uniform(2, 7))
    assert u[5] == (py_at(key, 5) >> 11) * 2.0 ** -53
