"""The synthetic input generator: counter-based, so a tensor is the same on
any device.  Pinned to the published SplitMix64 definition (a state advanced
by the golden-ratio increment, then the three-step xor-shift-multiply
finaliser), written here in plain Python integers; then the properties the
recipe states."""
import math

import numpy as np
import pytest
import torch

from decode_gemm_exp_amd import synth

M64 = (1 << 64) - 1


def splitmix64(state: int) -> int:
    """next() of SplitMix64 from `state` (returns the output)."""
    z = (state + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_draws_are_splitmix64():
    # element i of a stream with key K is next() from state K + i * gamma
    key = synth._key(synth.SEED_BASE, 3, 1)
    got = synth._draws(key, 0, 64, "cpu").numpy().view(np.uint64)
    for i in range(64):
        state = (key + i * 0x9E3779B97F4A7C15) & M64
        assert int(got[i]) == splitmix64(state), i
    # a window further on gives the same elements as the whole stream
    tail = synth._draws(key, 40, 24, "cpu").numpy().view(np.uint64)
    assert np.array_equal(tail, got[40:])


def test_normal_draws():
    z = synth._normal(synth._key(1, 2, 1), synth._key(1, 2, 2), 1 << 20, "cpu").numpy()
    assert abs(z.mean()) < 5 / 1024
    assert abs(z.std() - 1.0) < 5 / 1024
    # tails of a normal: P(|z| > 3) = 0.0027
    assert abs((np.abs(z) > 3).mean() - 0.0027) < 0.0005


def test_outliers_exact_count_and_scale():
    rows, cols, frac, shift = 64, 512, 0.003, 10
    plain = synth.weights(rows, cols, 0.02, 0.0, 0, seed=11).float().numpy()
    w = synth.weights(rows, cols, 0.02, frac, shift, seed=11).float().numpy()
    moved = np.nonzero(plain != w)[0] if plain.ndim == 1 else np.argwhere(plain != w)
    assert len(moved) == round(frac * rows * cols)
    r, c = moved[:, 0], moved[:, 1]
    assert np.array_equal(w[r, c], plain[r, c] * 2.0 ** shift)


def test_floyd_sample_distinct_and_uniform():
    pos = synth._floyd(synth._key(5, 6, 3), 1000, 500)
    assert len(set(pos.tolist())) == 500 and pos.min() >= 0 and pos.max() < 1000
    # every position is equally likely: 200 draws of 10 from 40, counts per position
    counts = np.zeros(40)
    for t in range(200):
        counts[synth._floyd(synth._key(9, t, 3), 40, 10)] += 1
    assert counts.min() > 20 and counts.max() < 80   # mean 50


def test_activations_and_bits_shapes():
    x = synth.activations(3, 256, seed=4)
    assert x.dtype == torch.bfloat16 and x.shape == (3, 256)
    b = synth.random_bits(8, 64, seed=4).view(torch.int16).numpy().view(np.uint16)
    assert b.shape == (8, 64) and len(np.unique(b)) > 400


@pytest.mark.gpu
def test_device_and_host_draws_identical():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    for fn in (lambda d: synth.weights(1000, 4096, 0.02, 0.0005, 10, seed=21, device=d),
               lambda d: synth.activations(7, 8192, seed=22, device=d),
               lambda d: synth.random_bits(33, 512, seed=23, device=d),
               lambda d: synth.fp8_weights(300, 1024, seed=24, device=d)):
        a = fn("cpu")
        b = fn("cuda:0").cpu()
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    wl = synth.WORKLOADS["gate8b"]
    a = synth.workload_weights(wl, 0, device="cpu")
    b = synth.workload_weights(wl, 0, device="cuda:0").cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
