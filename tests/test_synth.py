"""Host checks of the seeded input generators (no method arithmetic lives there)."""

import math

import numpy as np
import torch

import synth


def test_bf16_round_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(10000).astype(np.float32) * 3,
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, np.inf, -np.inf, 1e-40, -1e-40,
                  1.00390625, 1.01171875, 1.0078125 + 2 ** -24], np.float32),  # ties & subnormals
    ])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_frames_reproducible_and_distinct():
    a = synth.frame_block(3, 2, 5, 2, 10, 8, 0.5)
    b = synth.frame_block(3, 2, 5, 2, 10, 8, 0.5)
    c = synth.frame_block(3, 2, 6, 2, 10, 8, 0.5)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert a.dtype == np.float32


def test_top_k_counts():
    assert [synth.top_k_count(f, 220) for f in (0.125, 0.25, 0.5, 1.0)] == [28, 55, 110, 220]
    assert synth.top_k_count(0.25, 74) == 19
    assert synth.top_k_count(0.25, 147) == 37
    assert synth.top_k_count(0.001, 5) == 1


def test_wan_layer_shapes():
    wl = synth.WORKLOADS["wan_layer_bf16"]
    d = synth.wan_layer_inputs(1)
    assert d["q"].shape == (12, 4680, 128) and d["q"].dtype == np.uint16
    assert d["k"].shape == (12, 18720, 128)
    assert (d["ev_lo"], d["ev_hi"], d["win_lo"], d["win_hi"]) == (0, 4680, 4680, 18720)
    f = synth.bf16_bits_to_f32(d["q"][:2])
    assert abs(float(f.std()) - 1 / math.sqrt(wl.head_dim)) < 2e-3


def test_planted_construction():
    pi = synth.planted_inputs(4, 0.125)
    assert pi["top_k"] == 28
    s = pi["planted"]
    assert s.shape == (12, 74, 28)
    assert np.all(np.diff(s, axis=-1) > 0)
    assert s.min() >= 0 and s.max() < 220


def test_long_stream_drift():
    ls = synth.LongStream(2)
    assert np.all(ls.drift[0] == 0)
    step = np.diff(ls.drift, axis=0)
    assert abs(float(step.std()) - 0.05) < 0.005
    k0 = synth.bf16_bits_to_f32(ls.frame("k", 100))
    assert np.allclose(k0.mean(axis=1), ls.drift[100], atol=0.01)
