"""GPU parity against the oracle on the five workloads.

tiny and small run whole. For large, long and stress the oracle would need
minutes of float64 work on the host, so they run as seeded slices that keep
the workload's hidden width, full vocabulary, shard count and distributions
with fewer tokens (a ragged 777, not a tile multiple); the full-size runs are
checked row by row in test_gpu_zfullsize.
"""
import pytest

import workloads
from gpu_support import compare, oracle_for, run_lce, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_workload_parity(name):
    say("workload", name)
    b = workloads.make(name)
    gpu = run_lce(*to_device(b))
    compare(gpu, oracle_for(b), name)


def test_large_width_two_token_chunks():
    """The large workload's H, V and P with N = 16384 + 300 tokens: the backward
    runs two token chunks and two vocabulary chunks per shard (the fp32 dW of a
    shard accumulates over the token chunks), compared element by element with
    the oracle (about 5e13 float64 flops on the host)."""
    w = workloads.WORKLOADS["large"].with_tokens(16384 + 300)
    say("workload slice", w.name, "two token chunks at H =", w.hidden)
    b = workloads.make(w)
    gpu = run_lce(*to_device(b))
    say("oracle on the host ...")
    compare(gpu, oracle_for(b), w.name)


@pytest.mark.parametrize("name", ["large", "long", "stress"])
def test_workload_slice_parity(name):
    w = workloads.WORKLOADS[name].with_tokens(777)
    say("workload slice", w.name)
    b = workloads.make(w)
    gpu = run_lce(*to_device(b))
    compare(gpu, oracle_for(b), w.name)
