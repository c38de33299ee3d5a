"""The oracle against torch's float64 cross_entropy + autograd on slices of the real workloads.

Each slice keeps the workload's hidden width, full vocabulary, shard count and
distributions and takes its first few tokens, so the oracle is pinned at the
magnitudes the GPU parity tests use (including logits beyond |z| = 100 on the
stress workload). No GPU.
"""
import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads


@pytest.mark.slow
@pytest.mark.parametrize("name,rows", [("small", 64), ("large", 8), ("long", 8), ("stress", 8)])
def test_oracle_matches_torch_on_workload_slice(name, rows):
    w = workloads.WORKLOADS[name]
    b = workloads.make(w.with_tokens(rows))
    x = oracle.bf16_to_f64(b.hidden)
    wt = oracle.bf16_to_f64(b.weight)
    pins.check_torch_reference(oracle, x, wt, b.targets, tol=1e-9, row_block=max(1, rows // 3))
    if name == "stress":
        assert np.max(np.abs(x @ wt.T)) > 100.0       # the stress regime really is reached


def test_ring_fold_matches_plain_on_tiny():
    b = workloads.make("tiny")
    x = oracle.bf16_to_f64(b.hidden)
    shards = [oracle.bf16_to_f64(s) for s in b.shards]
    plain = oracle.cross_entropy(x, np.concatenate(shards), b.targets)
    for order in ([0, 3, 2, 1], [2, 0, 3, 1]):
        rf = oracle.ring_fold(x, shards, order, b.targets)
        assert abs(rf.loss - plain.loss) <= 1e-13
        np.testing.assert_allclose(rf.d_weight, plain.d_weight, rtol=1e-10, atol=1e-16)
        np.testing.assert_allclose(rf.d_hidden, plain.d_hidden, rtol=1e-10, atol=1e-16)
