"""Seeded input generator: determinism, recipe and distributions (no GPU)."""
import numpy as np
import pytest

import workloads
from workloads import WORKLOADS, bf16_bits_as_float32, f32_to_bf16_bits


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-39, 65504.0], dtype=np.float32)
    got = bf16_bits_as_float32(f32_to_bf16_bits(vals))
    # 1+2^-8 is a tie between 1 and 1+2^-7: ties go to the even mantissa (1.0)
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == np.float32(1.0 + 2**-6)
    assert got[3] == 1.0 and got[4] == -2.5
    import torch
    ref = torch.tensor(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref, f32_to_bf16_bits(vals))


def test_tiny_deterministic_and_recipe():
    a, b = workloads.make("tiny"), workloads.make("tiny")
    assert a.digest() == b.digest()
    c = workloads.make("tiny", seed=1)
    assert c.digest()["hidden"] != a.digest()["hidden"]
    w = WORKLOADS["tiny"]
    assert a.hidden.shape == (256, 128) and a.weight.shape == (1024, 128) and a.targets.dtype == np.int32
    assert len(a.shards) == 4 and all(s.shape == (256, 128) for s in a.shards)
    assert np.all((a.targets >= 0) & (a.targets < w.vocab))
    x = bf16_bits_as_float32(a.hidden)
    assert abs(x.std() - 1.0) < 0.02 and abs(x.mean()) < 0.02
    ww = bf16_bits_as_float32(a.weight)
    assert abs(ww.std() - 0.02) < 0.001


def test_prefix_stability_of_rows():
    w = WORKLOADS["small"].with_dims(hidden=64, vocab=800, n_tokens=5000)
    full = workloads.make(w)
    part = workloads.make(w.with_tokens(4500))
    assert np.array_equal(full.hidden[:4500], part.hidden)
    assert np.array_equal(full.weight, part.weight)


def test_small_distributions():
    b = workloads.make("small")
    w = WORKLOADS["small"]
    x = bf16_bits_as_float32(b.hidden[:512]).astype(np.float64)
    rms = np.sqrt((x * x).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 0.01)          # rows RMS-normalised (bf16 rounding aside)
    ign = b.targets == -100
    assert ign.sum() == int(np.floor(0.05 * 4096 + 0.5))
    t = b.targets[~ign]
    # finite Zipf(1.1): the head mass matches the law
    cdf = workloads.zipf_cdf(w.vocab, 1.1)
    assert abs((t == 0).mean() - cdf[0]) < 0.03
    assert abs((t < 100).mean() - cdf[99]) < 0.03
    assert t.max() < w.vocab and t.min() >= 0
    ww = bf16_bits_as_float32(b.weight[:2000])
    assert abs(ww.std() - 0.02) < 0.0005


def test_stress_shape_and_ignore_count():
    w = WORKLOADS["stress"]
    t = workloads.make_targets(w, 0)
    assert t.shape == (131071,)
    assert (t == -100).sum() == int(np.floor(0.1 * 131071 + 0.5))
    assert w.vocab % w.n_shards == 0 and w.shard_rows == 9496


@pytest.mark.parametrize("name", workloads.ORDER)
def test_every_workload_divides(name):
    w = WORKLOADS[name]
    assert w.vocab % w.n_shards == 0
